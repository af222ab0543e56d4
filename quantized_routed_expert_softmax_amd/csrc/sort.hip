// sort.hip — stable counting sort of the routed (token, j) pairs by expert and
// the pass table (hit experts in ascending id, at most P per pass).
//
// Sources: "POC: Experts offload", commit messages (sorted prefill runs 64
// experts at a time, so a prompt that routes to every expert stays bounded);
// "RFC: stream MoE experts from disk in from_pretrained", How the prototype
// works, Prefill (a long prompt routes to nearly every expert; they run through
// the sorted gather in groups of 64).
//
// Integer-only and deterministic: counts come from integer atomics (order-free),
// a pair's place is offsets[e] + (pairs of e in earlier tiles) + (pairs of e
// earlier in its own tile), which is the stable order by pair id.
//   n <= 1024 : one block does everything (decode and small batches).
//   n >  1024 : tile kernel (per-tile counts and in-tile ranks), one block that
//               turns the counts into per-tile bases, offsets and the pass table,
//               and a scatter kernel with one thread per pair.
#include "../../include/moe.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTile = 256;
constexpr int kSmallMax = 1024;

// Inclusive scan over the 64 lanes of a wave (shuffles; integer, exact).
__device__ inline int wave_inclusive_scan(int v, int lane)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
    }
    return v;
}

// Exclusive scan of s[0..E) in place over a 1024-thread block (16 waves): scan
// within waves, then the 16 wave totals; returns the total.  s_tmp needs 16 ints.
__device__ int block_exclusive_scan(int* s, int E, int* s_tmp)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int v = tid < E ? s[tid] : 0;
    const int inc = wave_inclusive_scan(v, lane);
    if (lane == 63) s_tmp[wave] = inc;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        const int t = s_tmp[w];
        before += w < wave ? t : 0;
        total += t;
    }
    if (tid < E) s[tid] = before + inc - v;
    __syncthreads();
    return total;
}

// Offsets, pass table and hit list from per-expert counts (s_cnt, length E),
// leaving exclusive offsets in s_cnt.  Runs on a full 1024-thread block.
__device__ void write_offsets_and_passes(int* s_cnt, int* s_tmp, int* s_hit, int E, int P,
                                         int32_t* offsets, int32_t* pass_table)
{
    const int tid = threadIdx.x;
    const int cnt = tid < E ? s_cnt[tid] : 0;
    if (tid < E) s_hit[tid] = cnt > 0 ? 1 : 0;
    __syncthreads();
    const int n_valid = block_exclusive_scan(s_cnt, E, s_tmp);
    const int n_hit = block_exclusive_scan(s_hit, E, s_tmp);
    if (tid < E) offsets[tid] = s_cnt[tid];
    if (tid == 0) offsets[E] = n_valid;
    // hit list: expert tid goes to position s_hit[tid] when hit
    if (tid < E) {
        pass_table[2 + tid] = -1;
    }
    __syncthreads();
    if (tid < E && cnt > 0) pass_table[2 + s_hit[tid]] = tid;
    const int n_pass_max = (E + P - 1) / P;
    const int n_pass = (n_hit + P - 1) / P;
    if (tid == 0) {
        pass_table[0] = n_hit;
        pass_table[1] = n_pass;
    }
    if (tid <= n_pass_max) {
        const int start = tid * P;
        pass_table[2 + E + tid] = start < n_hit ? start : n_hit;
    }
}

__global__ __launch_bounds__(1024) void sort_small_kernel(const int32_t* __restrict__ ids, int n,
                                                          int E, int P, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ pass_table,
                                                          uint32_t* __restrict__ err)
{
    __shared__ int s_e[kSmallMax];
    __shared__ int s_cnt[1024];
    __shared__ int s_tmp[1024];
    __shared__ int s_hit[1024];
    const int tid = threadIdx.x;
    int e = -1;
    if (tid < n) {
        e = ids[tid];
        if (e < 0 || e >= E) {
            if (err) atomicOr(err, MOE_ERRW_BAD_ID);
            e = -1;
        }
    }
    s_e[tid] = e;
    s_cnt[tid] = 0;
    __syncthreads();
    if (e >= 0) atomicAdd(&s_cnt[e], 1);
    int rank = 0;
    if (e >= 0)
        for (int q = 0; q < tid; ++q) rank += (s_e[q] == e);
    __syncthreads();
    write_offsets_and_passes(s_cnt, s_tmp, s_hit, E, P, offsets, pass_table);
    if (e >= 0) sorted_pairs[s_cnt[e] + rank] = tid;
}

// Per tile of kTile pairs: expert counts (tile_counts[b][E]) and in-tile ranks.
__global__ __launch_bounds__(kTile) void sort_tile_kernel(const int32_t* __restrict__ ids, int n,
                                                          int E, int32_t* __restrict__ tile_counts,
                                                          int32_t* __restrict__ rank_out,
                                                          uint32_t* __restrict__ err)
{
    __shared__ int s_e[kTile];
    __shared__ int s_cnt[1024];
    const int tid = threadIdx.x;
    const int p = blockIdx.x * kTile + tid;
    for (int i = tid; i < E; i += kTile) s_cnt[i] = 0;
    int e = -1;
    if (p < n) {
        e = ids[p];
        if (e < 0 || e >= E) {
            if (err) atomicOr(err, MOE_ERRW_BAD_ID);
            e = -1;
        }
    }
    s_e[tid] = e;
    __syncthreads();
    if (e >= 0) atomicAdd(&s_cnt[e], 1);
    int rank = 0;
    if (e >= 0)
        for (int q = 0; q < tid; ++q) rank += (s_e[q] == e);
    if (p < n) rank_out[p] = rank;
    __syncthreads();
    int32_t* tc = tile_counts + (size_t)blockIdx.x * E;
    for (int i = tid; i < E; i += kTile) tc[i] = s_cnt[i];
}

// One block: per-expert running sums over tiles (tile_counts becomes the base of
// each expert within each tile), offsets and the pass table.
__global__ __launch_bounds__(1024) void sort_scan_kernel(int E, int P, int n_tiles,
                                                         int32_t* __restrict__ tile_counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ pass_table)
{
    __shared__ int s_cnt[1024];
    __shared__ int s_tmp[1024];
    __shared__ int s_hit[1024];
    const int tid = threadIdx.x;
    if (tid < E) {
        // running sum over tiles; 16 independent loads per round trip
        int run = 0;
        for (int b0 = 0; b0 < n_tiles; b0 += 16) {
            int v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                v[j] = b0 + j < n_tiles ? tile_counts[(size_t)(b0 + j) * E + tid] : 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (b0 + j < n_tiles) {
                    tile_counts[(size_t)(b0 + j) * E + tid] = run;  // tile base of expert tid
                    run += v[j];
                }
            }
        }
        s_cnt[tid] = run;
    }
    __syncthreads();
    write_offsets_and_passes(s_cnt, s_tmp, s_hit, E, P, offsets, pass_table);
}

// One thread per pair: place = offsets[e] + base of e in the pair's tile + rank in tile.
__global__ __launch_bounds__(kTile) void sort_scatter_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                             const int32_t* __restrict__ tile_base,
                                                             const int32_t* __restrict__ rank_in,
                                                             const int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted_pairs)
{
    const int p = blockIdx.x * kTile + threadIdx.x;
    if (p >= n) return;
    const int e = ids[p];
    if (e < 0 || e >= E) return;  // flagged by the tile kernel
    const int r = rank_in[p];
    sorted_pairs[offsets[e] + tile_base[(size_t)blockIdx.x * E + e] + r] = p;
}

}  // namespace

size_t sort_ws_bytes(int T, int k, int E)
{
    const int64_t n = (int64_t)T * k;
    if (n <= kSmallMax) return 0;
    const int64_t tiles = (n + kTile - 1) / kTile;
    return (size_t)(tiles * E + n) * sizeof(int32_t);
}

hipError_t launch_sort(const int32_t* ids, int T, int k, int E, int P, int32_t* offsets,
                       int32_t* sorted_pairs, int32_t* pass_table, void* ws, uint32_t* err,
                       hipStream_t s)
{
    const int n = T * k;
    if (n <= kSmallMax) {
        hipLaunchKernelGGL(sort_small_kernel, dim3(1), dim3(1024), 0, s, ids, n, E, P, offsets,
                           sorted_pairs, pass_table, err);
        return hipGetLastError();
    }
    const int tiles = (n + kTile - 1) / kTile;
    int32_t* tile_counts = (int32_t*)ws;
    int32_t* ranks = tile_counts + (size_t)tiles * E;
    hipLaunchKernelGGL(sort_tile_kernel, dim3(tiles), dim3(kTile), 0, s, ids, n, E, tile_counts,
                       ranks, err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(1024), 0, s, E, P, tiles, tile_counts, offsets,
                       pass_table);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sort_scatter_kernel, dim3(tiles), dim3(kTile), 0, s, ids, n, E, tile_counts, ranks,
                       offsets, sorted_pairs);
    return hipGetLastError();
}

}  // namespace moe
