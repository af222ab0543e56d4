// sort.hip — stable counting sort of the routed (token, j) pairs by expert and
// the pass table (hit experts in ascending id, at most P per pass).
//
// Sources: "POC: Experts offload", commit messages (the sorted prefill takes the
// hit experts 64 per batch, which bounds its memory even when a prompt touches
// all of them); "RFC: stream MoE experts from disk in from_pretrained", How the
// prototype works, Prefill (almost every expert is hit by a long prompt; the
// sorted gather processes them in batches of 64).
//
// Integer-only and deterministic: counts come from integer atomics (order-free),
// a pair's place is offsets[e] + (pairs of e in earlier tiles) + (pairs of e
// earlier in its own tile), which is the stable order by pair id.
//   n <= 1024 : one block does everything (decode and small batches).
//   n >  1024 : tile kernel (per-tile counts and in-tile ranks), then one block
//               per tile that sums the counts into totals and its tile's bases,
//               scans the totals into offsets (block 0 writes them and the pass
//               table) and places its tile's pairs: two launches.
// The MFMA path's permute of x rides along in extra workgroups of the first
// launch (it does not depend on the sort).
#include "../../include/moe.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTile = 256;
constexpr int kSmallMax = 1024;

// Dword q of x [T, H] bf16 in the P16 layout of the MFMA path: within each
// 32-input chunk, position 2i + h holds input i + 16h (the permute that rides
// along with the sort's first launch).
__device__ __forceinline__ void permute_dw(const uint16_t* __restrict__ x, int64_t n_dw,
                                           uint32_t* __restrict__ xp, int64_t q)
{
    if (q >= n_dw) return;
    const int64_t chunk = q >> 4;
    const int i = (int)(q & 15);
    const uint16_t* src = x + chunk * 32;
    xp[q] = (uint32_t)src[i] | ((uint32_t)src[i + 16] << 16);
}

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
// leaving exclusive offsets in s_cnt.  Runs on a full 1024-thread block; with
// offsets and pass_table null it only computes the offsets in s_cnt.
__device__ void write_offsets_and_passes(int* s_cnt, int* s_tmp, int* s_hit, int E, int P,
                                         int32_t* offsets, int32_t* pass_table)
{
    if (!offsets) {
        block_exclusive_scan(s_cnt, E, s_tmp);
        return;
    }
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
                                                          uint32_t* __restrict__ err,
                                                          const uint16_t* __restrict__ x, int64_t n_dw,
                                                          uint32_t* __restrict__ xp)
{
    __shared__ int s_e[kSmallMax];
    __shared__ int s_cnt[1024];
    __shared__ int s_tmp[1024];
    __shared__ int s_hit[1024];
    const int tid = threadIdx.x;
    if (blockIdx.x > 0) {  // workgroups past the first: the permute of x
        permute_dw(x, n_dw, xp, (int64_t)(blockIdx.x - 1) * 1024 + tid);
        return;
    }
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
                                                          uint32_t* __restrict__ err, int tiles,
                                                          const uint16_t* __restrict__ x, int64_t n_dw,
                                                          uint32_t* __restrict__ xp)
{
    __shared__ int s_e[kTile];
    __shared__ int s_cnt[1024];
    const int tid = threadIdx.x;
    if ((int)blockIdx.x >= tiles) {  // workgroups past the tiles: the permute of x
        permute_dw(x, n_dw, xp, (int64_t)(blockIdx.x - tiles) * kTile + tid);
        return;
    }
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

// One block per tile, after the tile kernel: every block sums the tile counts of
// all experts (the totals, and its own tile's base per expert: the counts of the
// tiles before it) and scans the totals into offsets itself, so no launch has
// to wait for a single scan block; block 0 also writes the offsets and the pass
// table.  Then each pair goes to offsets[e] + base of e in its tile + its rank in
// the tile.
__global__ __launch_bounds__(1024) void sort_place_kernel(const int32_t* __restrict__ ids, int n, int E, int P,
                                                          int n_tiles, const int32_t* __restrict__ tile_counts,
                                                          const int32_t* __restrict__ rank_in,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ pass_table,
                                                          int32_t* __restrict__ sorted_pairs)
{
    __shared__ int s_cnt[1024];
    __shared__ int s_tmp[1024];
    __shared__ int s_hit[1024];
    __shared__ int s_base[1024];
    const int tid = threadIdx.x, b = blockIdx.x;
    if (tid < E) {
        // 16 independent loads per round trip
        int run = 0, base = 0;
        for (int b0 = 0; b0 < n_tiles; b0 += 16) {
            int v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = b0 + j < n_tiles ? tile_counts[(size_t)(b0 + j) * E + tid] : 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (b0 + j == b) base = run;
                run += v[j];
            }
        }
        s_cnt[tid] = run;
        s_base[tid] = base;
    }
    __syncthreads();
    write_offsets_and_passes(s_cnt, s_tmp, s_hit, E, P, b == 0 ? offsets : nullptr,
                             b == 0 ? pass_table : nullptr);
    __syncthreads();
    if (tid < kTile) {
        const int p = b * kTile + tid;
        if (p < n) {
            const int e = ids[p];
            if (e >= 0 && e < E)  // (out-of-range ids are flagged by the tile kernel)
                sorted_pairs[s_cnt[e] + s_base[e] + rank_in[p]] = p;
        }
    }
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
                       hipStream_t s, const uint16_t* x_perm, int H, uint16_t* xp)
{
    const int n = T * k;
    const int64_t n_dw = x_perm ? (int64_t)T * H / 2 : 0;  // permute dwords riding along
    if (n <= kSmallMax) {
        const int64_t pb = (n_dw + 1023) / 1024;
        hipLaunchKernelGGL(sort_small_kernel, dim3((unsigned)(1 + pb)), dim3(1024), 0, s, ids, n, E, P, offsets,
                           sorted_pairs, pass_table, err, x_perm, n_dw, (uint32_t*)xp);
        return hipGetLastError();
    }
    const int tiles = (n + kTile - 1) / kTile;
    const int64_t pb = (n_dw + kTile - 1) / kTile;
    int32_t* tile_counts = (int32_t*)ws;
    int32_t* ranks = tile_counts + (size_t)tiles * E;
    hipLaunchKernelGGL(sort_tile_kernel, dim3((unsigned)(tiles + pb)), dim3(kTile), 0, s, ids, n, E, tile_counts,
                       ranks, err, tiles, x_perm, n_dw, (uint32_t*)xp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sort_place_kernel, dim3(tiles), dim3(1024), 0, s, ids, n, E, P, tiles, tile_counts, ranks,
                       offsets, pass_table, sorted_pairs);
    return hipGetLastError();
}

}  // namespace moe
