// worklist.hip -- document-local work list built on the GPU, sorted by
// decreasing cost (FLAMIA review section 6, Algorithm 2: items of a bounded
// number of queries from one document, cost estimated in visible key blocks,
// sorted across the packed row, built without host synchronisation).
//
// Forward items are (document, 128-query tile), cost = number of 64-key steps
// the tile visits.  Backward items are (document, key tile of 128 or 256
// keys), cost = number of 64-query tiles visited.  One 1024-thread workgroup performs a
// counting sort by cost: per-document item counts are scanned, every item
// finds its document by binary search and bumps a cost histogram, the
// histogram is scanned from the largest cost down, and items are scattered
// into their buckets (order inside a bucket is unspecified; it affects only
// scheduling, never results).  For the persistent backward it also decides
// how many of the costliest items are split into two tickets.
#include "device.hpp"
#include "kernels.hpp"

namespace flamia {

namespace {

constexpr int kThreads = 1024;

// Exclusive scan of v over the workgroup; returns the prefix, writes total.
__device__ int block_exclusive_scan(int v, int* s_tmp, int* total)
{
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    int x = v;
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    if (lane == 63) s_tmp[wid] = x;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int w = 0; w < kThreads / 64; ++w) {
            int c = s_tmp[w];
            s_tmp[w] = acc;
            acc += c;
        }
        s_tmp[kThreads / 64] = acc;
    }
    __syncthreads();
    int out = x - v + s_tmp[wid];
    *total = s_tmp[kThreads / 64];
    __syncthreads();
    return out;
}

__device__ __forceinline__ int item_cost(const WorklistArgs& a, int n, int m)
{
    const int steps64 = (n + 63) / 64;
    if (a.backward) {
        // query tiles of 64 visited by key tile m (keys [tile m, tile (m + 1)))
        return a.causal ? steps64 - (a.tile / 64) * m : steps64;
    }
    // 64-key steps visited by query tile m (queries [128 m, 128 m + 128))
    return a.causal ? (min(a.tile * (m + 1), n) + 63) / 64 : steps64;
}

// Sizes up to which the document offsets, the histogram and the bucket
// cursors live in LDS (48 KB), so that the phases meet through LDS instead
// of device memory; larger problems use the workspace arrays.
constexpr int kLdsEntries = 4096;

template <bool LDS>
__global__ __launch_bounds__(kThreads) void worklist_kernel(WorklistArgs a)
{
    __shared__ int s_tmp[kThreads / 64 + 1];
    __shared__ int s_arr[LDS ? 3 : 1][LDS ? kLdsEntries : 1];
    const int tid = threadIdx.x;
    const int32_t* cu = a.cu;
    int* doc_off = LDS ? s_arr[0] : a.doc_off;
    int* hist = LDS ? s_arr[1] : a.hist;
    int* cursor = LDS ? s_arr[2] : a.cursor;

    // 1. items per document, exclusive scan -> doc_off
    int carry = 0;
    for (int base = 0; base < a.B; base += kThreads) {
        const int b = base + tid;
        int c = 0;
        if (b < a.B) {
            const int n = cu[b + 1] - cu[b];
            c = (n + a.tile - 1) / a.tile;
        }
        int total;
        int pre = block_exclusive_scan(c, s_tmp, &total);
        if (b < a.B) doc_off[b] = carry + pre;
        carry += total;
    }
    if (tid == 0) doc_off[a.B] = carry;
    const int nitems = min(carry, a.max_items);
    for (int c = tid; c <= a.max_cost; c += kThreads) hist[c] = 0;
    __syncthreads();
    __threadfence_block();

    // 2. cost histogram
    for (int i = tid; i < nitems; i += kThreads) {
        int lo = 0, hi = a.B - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (doc_off[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        const int n = cu[lo + 1] - cu[lo];
        const int cost = min(item_cost(a, n, i - doc_off[lo]), a.max_cost);
        atomicAdd(&hist[cost], 1);
    }
    __syncthreads();
    __threadfence_block();

    // 3. bucket starts, largest cost first
    carry = 0;
    for (int base = 0; base <= a.max_cost; base += kThreads) {
        const int c = a.max_cost - (base + tid);  // descending cost
        const int v = c >= 0 ? hist[c] : 0;
        int total;
        int pre = block_exclusive_scan(v, s_tmp, &total);
        if (c >= 0) cursor[c] = carry + pre;
        carry += total;
    }
    __syncthreads();
    __threadfence_block();

    // 3b. (backward) items split in two, only when there are fewer than
    // eight tickets per workgroup (with more, the cost-ordered queue already
    // balances the grid and halves only add per-ticket work): those whose
    // tickets cost more than half of a workgroup's average share of all
    // tickets, i.e. cost c > Hkv sum(c) / (2 workgroups), and at least
    // split_min_cost (a half must outweigh the slots it writes and reads).
    // They are the leading buckets, so their number is the start of bucket
    // thr - 1 (read before the scatter moves the cursors); at most split_cap.
    int nsplit = 0;
    if (a.split_cap > 0 && (int64_t)nitems * a.split_hkv < 8 * (int64_t)a.split_wgs) {
        int part = 0;
        for (int c = tid; c <= a.max_cost; c += kThreads) part += c * hist[c];
        int total;
        (void)block_exclusive_scan(part, s_tmp, &total);
        const int64_t thr = max<int64_t>(max(a.split_min_cost, 2),
                                         (int64_t)a.split_hkv * total / (2 * (int64_t)a.split_wgs) + 1);
        nsplit = thr > a.max_cost ? 0 : min(cursor[thr - 1], a.split_cap);
    }

    // 4. scatter
    for (int i = tid; i < nitems; i += kThreads) {
        int lo = 0, hi = a.B - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (doc_off[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        const int m = i - doc_off[lo];
        const int n = cu[lo + 1] - cu[lo];
        const int cost = min(item_cost(a, n, m), a.max_cost);
        const int pos = atomicAdd(&cursor[cost], 1);
        a.items[2 * pos] = lo;
        a.items[2 * pos + 1] = m;
    }
    // count[1]: the ticket counter of the persistent backward, taken from 0;
    // count[2]: the number of leading items split in two
    if (tid == 0) {
        a.count[0] = nitems;
        a.count[1] = 0;
        a.count[2] = nsplit;
    }
}

}  // namespace

hipError_t launch_worklist(const WorklistArgs& a, hipStream_t stream)
{
    if (a.B + 1 <= kLdsEntries && a.max_cost + 1 <= kLdsEntries)
        hipLaunchKernelGGL(worklist_kernel<true>, dim3(1), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(worklist_kernel<false>, dim3(1), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace flamia
