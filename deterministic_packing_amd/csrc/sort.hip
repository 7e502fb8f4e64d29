// sort.hip — compaction of kept documents, Philox4x32-10 shuffle keys, and a
// stable LSD radix sort of the kept documents by (group, key64).
//
// NeuronSpark-Trainer README, Concepts: a file's documents are shuffled.  The
// shuffle here is counter-based: key64(d) = x1·2^32 + x0 of
// Philox4x32-10(counter = (d lo, d hi, 0x53485546, 0), key = (seed lo, seed hi))
// (Salmon et al., SC'11), so it depends only on the seed and the input index d,
// never on rank, world or launch shape.  Kept documents enter the sort in
// input order and every pass is stable.  The radix passes order by
// (group, key64 >> 32) only; runs that tie there (rare: about n²/2^33 pairs
// for n documents of a group) are then ordered by the low 32 key bits with a
// stable insertion sort, which leaves ties of key64 in input order, so the
// result is the order by (group, key64, d).
#include "dp_common.h"

namespace dp {
namespace {

constexpr int RB = 256;             // threads per block
constexpr int RI = 8;               // rounds per tile
constexpr int RTILE = RB * RI;      // elements per tile

__global__ __launch_bounds__(256) void k_compact_keys(Plan p, uint64_t* key, uint32_t* val) {
    const uint64_t d = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (d >= p.n_docs || !p.keep[d]) return;
    const uint32_t at = p.kept_pos[d];
    val[at] = (uint32_t)d;
    key[at] = philox_key64((uint32_t)d, (uint32_t)(d >> 32), 0x53485546u, 0u, (uint32_t)p.seed,
                           (uint32_t)(p.seed >> 32));
}

template <bool GROUP>
__device__ inline uint32_t digit_of(uint64_t key, uint32_t val, const uint32_t* group, int shift) {
    if (GROUP) return (group[val] >> shift) & 0xFFu;
    return (uint32_t)(key >> shift) & 0xFFu;
}

template <bool GROUP>
__global__ __launch_bounds__(RB) void k_hist(const uint64_t* key, const uint32_t* val, const uint32_t* group,
                                             uint64_t n, int shift, uint32_t* hist, uint32_t nb) {
    __shared__ uint32_t h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const uint64_t base = (uint64_t)blockIdx.x * RTILE;
    for (int r = 0; r < RI; ++r) {
        const uint64_t i = base + (uint64_t)r * RB + threadIdx.x;
        if (i < n) atomicAdd(&h[digit_of<GROUP>(GROUP ? 0 : key[i], GROUP ? val[i] : 0, group, shift)], 1u);
    }
    __syncthreads();
    hist[(uint64_t)threadIdx.x * nb + blockIdx.x] = h[threadIdx.x];
}

// Stable scatter: element i of the tile lands at
//   offset[digit][tile] + (# earlier elements of the tile with the same digit).
// Within a round of 256 elements the earlier same-digit lanes of a wave come
// from ballots over the 8 digit bits; earlier waves and rounds from LDS counts.
template <bool GROUP>
__global__ __launch_bounds__(RB) void k_scatter(const uint64_t* key_in, const uint32_t* val_in,
                                                const uint32_t* group, uint64_t n, int shift,
                                                const uint32_t* hofs, uint32_t nb, uint64_t* key_out,
                                                uint32_t* val_out, uint32_t* err) {
    __shared__ uint32_t running[256];
    __shared__ uint32_t wcount[RB / WAVE][256];
    const int t = threadIdx.x, wid = t / WAVE, lane = t & (WAVE - 1);
    running[t] = hofs[(uint64_t)t * nb + blockIdx.x];
#pragma unroll
    for (int w = 0; w < RB / WAVE; ++w) wcount[w][t] = 0;
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
    const uint64_t base = (uint64_t)blockIdx.x * RTILE;
    for (int r = 0; r < RI; ++r) {
        const uint64_t i = base + (uint64_t)r * RB + t;
        const bool valid = i < n;
        uint64_t k = 0;
        uint32_t v = 0, dg = 0;
        if (valid) {
            k = key_in[i];
            v = val_in[i];
            dg = digit_of<GROUP>(k, v, group, shift);
        }
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (dg >> b) & 1u;
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const uint32_t rank = (uint32_t)__popcll(peers & lt_mask);
        if (valid && rank == 0) wcount[wid][dg] = (uint32_t)__popcll(peers);
        __syncthreads();
        if (valid) {
            uint32_t dst = running[dg] + rank;
            for (int w = 0; w < wid; ++w) dst += wcount[w][dg];
            if (dst < n) {
                key_out[dst] = k;
                val_out[dst] = v;
            } else {
                atomicOr(err, ERR_INTERNAL);
            }
        }
        __syncthreads();
        uint32_t add = 0;
#pragma unroll
        for (int w = 0; w < RB / WAVE; ++w) {
            add += wcount[w][t];
            wcount[w][t] = 0;
        }
        running[t] += add;
        __syncthreads();
    }
}

// Random read order of each source's cycle windows (NeuronSpark-Trainer
// README, Concepts: the trainer reads each source's windows of a segment in a
// random order; a segment read as a cycle).  Element e of the cycle's windows
// is source s's i-th window; key64 = x1·2^32 + x0 of Philox4x32-10(counter =
// (i, s, cycle, 0x57494E44), key = seed); sorted by (s, key64, e).
__global__ __launch_bounds__(256) void k_window_keys(Plan p, uint32_t cycle, uint64_t total) {
    const uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total) return;
    uint32_t lo = 0, hi = p.S;  // source: the last s with perm_start[s] <= e
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (p.perm_start[mid] <= e) lo = mid;
        else hi = mid - 1;
    }
    const uint32_t s = lo;
    const uint32_t i = (uint32_t)(e - p.perm_start[s]);
    p.wkey[0][e] = philox_key64(i, s, cycle, 0x57494E44u, (uint32_t)p.seed, (uint32_t)(p.seed >> 32));
    p.wval[0][e] = (uint32_t)e;
    p.wgroup[e] = s;
}

__global__ __launch_bounds__(256) void k_perm_out(Plan p, const uint32_t* sorted, uint64_t total) {
    const uint64_t r = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= total) return;
    const uint32_t e = sorted[r];
    p.perm[r] = (uint32_t)(e - p.perm_start[p.wgroup[e]]);
}

// Orders each run of equal (group, key64 >> 32) by the low 32 key bits; the
// thread at a run's first element sorts the run (insertion sort, stable).
// Other threads only read the high key bits and groups, which the sort of a
// run does not change.
__global__ __launch_bounds__(256) void k_tie_fix(uint64_t* key, uint32_t* val, const uint32_t* group, uint64_t n) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t hi = (uint32_t)(key[i] >> 32), g = group[val[i]];
    auto same = [&](uint64_t j) { return (uint32_t)(key[j] >> 32) == hi && group[val[j]] == g; };
    if (i > 0 && same(i - 1)) return;     // not the first element of its run
    if (i + 1 >= n || !same(i + 1)) return;  // a run of one
    uint64_t end = i + 2;
    while (end < n && same(end)) ++end;
    for (uint64_t a = i + 1; a < end; ++a) {
        const uint64_t k = key[a];
        const uint32_t v = val[a];
        uint64_t b = a;
        while (b > i && (uint32_t)key[b - 1] > (uint32_t)k) {
            key[b] = key[b - 1];
            val[b] = val[b - 1];
            --b;
        }
        key[b] = k;
        val[b] = v;
    }
}

}  // namespace

void launch_keep_scan(Plan& p, hipStream_t st) {
    scan_keep_u32(p.keep, p.n_docs, p.kept_pos, p.hist, st);
    const uint64_t blocks = (p.n_docs + 255) / 256;
    hipLaunchKernelGGL(k_compact_keys, dim3((uint32_t)blocks), dim3(256), 0, st, p, p.key[0], p.val[0]);
    DP_HIP(hipGetLastError());
}

// Stable sort of n (key64, val) pairs by (group[val], key64, input order),
// ping-ponging between buffers 0 and 1; returns the buffer that holds the
// result.  group values are < G.
uint32_t sort_pairs(uint64_t* const key[2], uint32_t* const val[2], const uint32_t* group, uint64_t n, uint32_t G,
                    uint32_t* hist_ws, uint32_t* err, hipStream_t st) {
    const uint32_t nb = (uint32_t)((n + RTILE - 1) / RTILE);
    // hist holds [256·nb] counts followed by [256·nb + 1] scanned offsets and the scan's temp
    uint32_t* hist = hist_ws;
    uint32_t* hofs = hist_ws + 256ull * nb + 1;
    void* tmp = hofs + 256ull * nb + 2;
    int cur = 0;
    auto pass = [&](bool group_pass, int shift) {
        if (nb == 0) return;
        if (group_pass)
            hipLaunchKernelGGL(k_hist<true>, dim3(nb), dim3(RB), 0, st, key[cur], val[cur], group, n, shift, hist, nb);
        else
            hipLaunchKernelGGL(k_hist<false>, dim3(nb), dim3(RB), 0, st, key[cur], val[cur], group, n, shift, hist,
                               nb);
        scan_u32(hist, 256ull * nb, hofs, tmp, st);
        if (group_pass)
            hipLaunchKernelGGL(k_scatter<true>, dim3(nb), dim3(RB), 0, st, key[cur], val[cur], group, n, shift, hofs,
                               nb, key[cur ^ 1], val[cur ^ 1], err);
        else
            hipLaunchKernelGGL(k_scatter<false>, dim3(nb), dim3(RB), 0, st, key[cur], val[cur], group, n, shift, hofs,
                               nb, key[cur ^ 1], val[cur ^ 1], err);
        DP_HIP(hipGetLastError());
        cur ^= 1;
    };
    for (int shift = 32; shift < 64; shift += 8) pass(false, shift);
    for (int shift = 0; G > 1 && shift < 32 && ((G - 1) >> shift) != 0; shift += 8) pass(true, shift);
    if (n > 1) {
        hipLaunchKernelGGL(k_tie_fix, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, st, key[cur], val[cur], group,
                           n);
        DP_HIP(hipGetLastError());
    }
    return (uint32_t)cur;
}

// requires p.n_kept (host) to be set
void launch_sort(Plan& p, hipStream_t st) {
    p.sort_buf = sort_pairs(p.key, p.val, p.group, p.n_kept, p.G, p.hist, p.err, st);
}

// requires perm_start (device) for the cycle; total = U·B
void launch_read_order(Plan& p, uint32_t cycle, uint64_t total, hipStream_t st) {
    if (total == 0) return;
    const uint32_t blocks = (uint32_t)((total + 255) / 256);
    hipLaunchKernelGGL(k_window_keys, dim3(blocks), dim3(256), 0, st, p, cycle, total);
    DP_HIP(hipGetLastError());
    const uint32_t buf = sort_pairs(p.wkey, p.wval, p.wgroup, total, p.S, p.hist, p.err, st);
    hipLaunchKernelGGL(k_perm_out, dim3(blocks), dim3(256), 0, st, p, (const uint32_t*)p.wval[buf], total);
    DP_HIP(hipGetLastError());
}

// workspace for the sort's histogram, offsets and scan temp, in uint32 words
uint64_t sort_hist_words(uint64_t n_docs) {
    const uint64_t nb = (n_docs + RTILE - 1) / RTILE + 1;
    return 256ull * nb * 2 + 4 + (scan_temp_bytes(256ull * nb) + 3) / 4 + 16;
}

}  // namespace dp
