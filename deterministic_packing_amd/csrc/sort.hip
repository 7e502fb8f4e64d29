// sort.hip — compaction of kept documents, Philox4x32-10 shuffle keys, and a
// sort of the kept documents by (group, key64, input index).
//
// NeuronSpark-Trainer README, Concepts: a file's documents are shuffled.  The
// shuffle here is counter-based: key64(d) = x1·2^32 + x0 of
// Philox4x32-10(counter = (d lo, d hi, 0x53485546, 0), key = (seed lo, seed hi))
// (Salmon et al., SC'11), so it depends only on the seed and the input index d,
// never on rank, world or launch shape.
//
// The sort is a distribution sort that relies on the keys' high bits being
// uniform (they are Philox outputs): a group of n elements is cut into 2^b
// buckets by the top b key bits, b the least with n >> b <= 4, so a bucket
// holds about two to four elements; elements reach their bucket through
// atomic tickets (in no particular order) and one thread per bucket then
// orders it by (key64, input index) with an insertion sort.  The result is the
// unique order by (group, key64, input index), whatever the tickets were.
#include "dp_common.h"

namespace dp {
namespace {

constexpr uint32_t LDS_GROUPS = 8192;  // group counts kept in LDS up to this many groups

// Adds 1 to bin g of every lane with c: a wavefront whose counting lanes share
// one group adds their number once, others lane by lane.
__device__ __forceinline__ void count_group(uint32_t* bins, bool c, uint32_t g) {
    const uint64_t m = __ballot(c);
    if (!m) return;
    const uint32_t g0 = (uint32_t)__builtin_amdgcn_readlane((int)g, (int)__builtin_ctzll(m));
    if (__all(!c || g == g0)) {
        if (lane_id() == (uint32_t)__builtin_ctzll(m)) atomicAdd(&bins[g0], (uint32_t)__popcll(m));
    } else if (c) {
        atomicAdd(&bins[g], 1u);
    }
}

// Compaction of the kept documents with their keys; it also counts the kept
// documents of each group into gcount (zeroed when the plan starts).  A
// grid of at most 1,024 blocks strides over the documents; with G <=
// LDS_GROUPS each block counts in LDS (G words of dynamic LDS) and adds its
// nonzero bins at the end, so few global atomics meet on one counter (with one
// thread per document and a block's bins added per block, or a wavefront's
// count added directly, the compaction measured 1.4x and 6.7x slower on the
// pre-train corpus: atomics on a few counters serialize).
__global__ __launch_bounds__(256) void k_compact_keys(Plan p, uint64_t* key, uint32_t* val, uint32_t* gcount,
                                                      uint32_t lds) {
    extern __shared__ uint32_t h[];
    if (lds) {
        for (uint32_t g = threadIdx.x; g < p.G; g += blockDim.x) h[g] = 0;
        __syncthreads();
    }
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t d0 = (uint64_t)blockIdx.x * blockDim.x; d0 < p.n_docs; d0 += stride) {
        const uint64_t d = d0 + threadIdx.x;
        const bool kept = d < p.n_docs && p.keep[d];
        const uint32_t g = kept ? p.group[d] : 0u;
        if (lds) count_group(h, kept, g);  // (two calls: LDS and global atomics, not flat ones)
        else count_group(gcount, kept, g);
        if (kept) {
            const uint32_t at = p.kept_pos[d];
            val[at] = (uint32_t)d;
            key[at] = philox_key64((uint32_t)d, (uint32_t)(d >> 32), 0x53485546u, 0u, (uint32_t)p.seed,
                                   (uint32_t)(p.seed >> 32));
        }
    }
    if (lds) {
        __syncthreads();
        for (uint32_t g = threadIdx.x; g < p.G; g += blockDim.x)
            if (h[g]) atomicAdd(&gcount[g], h[g]);
    }
}

// buckets of a group of n elements: 2^b, b the least with n >> b <= 4
__device__ __forceinline__ uint32_t bucket_bits(uint32_t n) {
    uint32_t b = 0;
    while ((n >> b) > 4u) ++b;
    return b;
}


// gcount[g] += elements of group g (gcount zeroed before); with G <=
// LDS_GROUPS the block counts in LDS first (G words of dynamic LDS)
__global__ __launch_bounds__(256) void k_group_count(const uint32_t* val, const uint32_t* group, uint64_t n,
                                                     uint32_t G, uint32_t* gcount) {
    extern __shared__ uint32_t h[];
    const bool lds = G <= LDS_GROUPS;
    if (lds) {
        for (uint32_t g = threadIdx.x; g < G; g += blockDim.x) h[g] = 0;
        __syncthreads();
    }
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i0 = (uint64_t)blockIdx.x * blockDim.x; i0 < n; i0 += stride) {
        const uint64_t i = i0 + threadIdx.x;
        const uint32_t g = i < n ? group[val[i]] : 0xFFFFFFFFu;
        // kept documents come grouped: a wavefront of one group adds once
        const uint32_t g0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)g);
        const bool one_group = __all(g == g0);  // every lane below n (g0 is then a group)
        if (one_group && g0 != 0xFFFFFFFFu) {
            if (lane_id() == 0) {
                if (lds) atomicAdd(&h[g0], (uint32_t)WAVE);
                else atomicAdd(&gcount[g0], (uint32_t)WAVE);
            }
        } else if (i < n) {
            if (lds) atomicAdd(&h[g], 1u);
            else atomicAdd(&gcount[g], 1u);
        }
    }
    if (lds) {
        __syncthreads();
        for (uint32_t g = threadIdx.x; g < G; g += blockDim.x)
            if (h[g]) atomicAdd(&gcount[g], h[g]);
    }
}

// gbase[g] = first bucket of group g (exclusive prefix of 2^b_g), gbase[G] =
// the buckets in use; one block of 1,024 threads, each over a run of groups
__global__ __launch_bounds__(1024) void k_bucket_base(const uint32_t* gcount, uint32_t G, uint32_t* gbase) {
    __shared__ uint32_t part[1024];
    const uint32_t per = (G + 1023) / 1024, g0 = threadIdx.x * per, g1 = min(G, g0 + per);
    uint32_t sum = 0;
    for (uint32_t g = g0; g < g1; ++g) sum += 1u << bucket_bits(gcount[g]);
    part[threadIdx.x] = sum;
    __syncthreads();
    for (uint32_t o = 1; o < 1024; o <<= 1) {  // inclusive scan of the runs' sums
        const uint32_t y = threadIdx.x >= o ? part[threadIdx.x - o] : 0u;
        __syncthreads();
        part[threadIdx.x] += y;
        __syncthreads();
    }
    uint32_t at = part[threadIdx.x] - sum;
    for (uint32_t g = g0; g < g1; ++g) {
        gbase[g] = at;
        at += 1u << bucket_bits(gcount[g]);
    }
    if (threadIdx.x == 1023) gbase[G] = part[1023];
}

constexpr uint32_t BASE_LDS_GROUPS = 1024;  // up to this many groups every block finds the bucket bases itself

// element i's bucket and its ticket in it (bcount zeroed before).  LDS_BASE
// (G <= BASE_LDS_GROUPS): each block first computes the groups' first buckets
// in LDS, as k_bucket_base does, and gbase is not read; else from gbase.
template <bool LDS_BASE>
__global__ __launch_bounds__(256) void k_bucket_count(const uint64_t* key, const uint32_t* val, const uint32_t* group,
                                                      uint64_t n, uint32_t G, const uint32_t* gcount,
                                                      const uint32_t* gbase, uint32_t* bcount, uint32_t* bucket,
                                                      uint32_t* ticket) {
    __shared__ uint32_t sbase[LDS_BASE ? BASE_LDS_GROUPS : 1];
    __shared__ uint32_t part[LDS_BASE ? 256 : 1];
    if constexpr (LDS_BASE) {
        const uint32_t per = (G + 255) / 256, g0 = threadIdx.x * per, g1 = min(G, g0 + per);
        uint32_t sum = 0;
        for (uint32_t g = g0; g < g1; ++g) {
            sbase[g] = 1u << bucket_bits(gcount[g]);
            sum += sbase[g];
        }
        part[threadIdx.x] = sum;
        __syncthreads();
        for (uint32_t o = 1; o < 256; o <<= 1) {  // inclusive scan of the runs' sums
            const uint32_t y = threadIdx.x >= o ? part[threadIdx.x - o] : 0u;
            __syncthreads();
            part[threadIdx.x] += y;
            __syncthreads();
        }
        uint32_t at = part[threadIdx.x] - sum;
        for (uint32_t g = g0; g < g1; ++g) {
            const uint32_t w = sbase[g];
            sbase[g] = at;
            at += w;
        }
        __syncthreads();
    }
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t g = group[val[i]];
    const uint32_t b = bucket_bits(gcount[g]);
    const uint32_t hi = (uint32_t)(key[i] >> 32);
    const uint32_t bk = (LDS_BASE ? sbase[g] : gbase[g]) + (b ? hi >> (32u - b) : 0u);
    bucket[i] = bk;
    ticket[i] = atomicAdd(&bcount[bk], 1u);
}

__global__ __launch_bounds__(256) void k_bucket_scatter(const uint64_t* key, const uint32_t* val, uint64_t n,
                                                        const uint32_t* bucket, const uint32_t* ticket,
                                                        const uint32_t* boff, uint64_t* key_out, uint32_t* val_out) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t at = boff[bucket[i]] + ticket[i];
    key_out[at] = key[i];
    val_out[at] = val[i];
}

constexpr uint32_t BMAX = 16;  // bucket sizes sorted in registers

__device__ __forceinline__ void cmpx(uint64_t& ka, uint32_t& va, uint64_t& kb, uint32_t& vb) {
    const bool sw = ka > kb || (ka == kb && va > vb);
    const uint64_t k = sw ? kb : ka, k2 = sw ? ka : kb;
    const uint32_t v = sw ? vb : va, v2 = sw ? va : vb;
    ka = k; kb = k2; va = v; vb = v2;
}

// one thread per bucket: [boff[b], boff[b+1]) ordered by (key64, val).  Up to
// BMAX elements are loaded at once, padded with the largest pair and sorted by
// an odd-even transposition network in registers; a larger bucket (rare: a
// bucket averages 2-4 elements) is sorted in place by insertion, as is every
// bucket with insertion_only (a test option, so that path is exercised).
__global__ __launch_bounds__(256) void k_bucket_sort(uint64_t* key, uint32_t* val, const uint32_t* boff, uint64_t nb,
                                                     uint32_t insertion_only) {
    const uint64_t b = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nb) return;
    const uint32_t lo = boff[b], hi = boff[b + 1];
    const uint32_t m = hi - lo;
    if (m < 2) return;
    if (m <= BMAX && !insertion_only) {
        uint64_t k[BMAX];
        uint32_t v[BMAX];
#pragma unroll
        for (uint32_t j = 0; j < BMAX; ++j) {
            k[j] = j < m ? key[lo + j] : ~0ull;
            v[j] = j < m ? val[lo + j] : ~0u;
        }
#pragma unroll
        for (uint32_t r = 0; r < BMAX; ++r)
#pragma unroll
            for (uint32_t j = r & 1u; j + 1 < BMAX; j += 2) cmpx(k[j], v[j], k[j + 1], v[j + 1]);
#pragma unroll
        for (uint32_t j = 0; j < BMAX; ++j)
            if (j < m) {
                key[lo + j] = k[j];
                val[lo + j] = v[j];
            }
        return;
    }
    for (uint32_t a = lo + 1; a < hi; ++a) {
        const uint64_t k = key[a];
        const uint32_t v = val[a];
        uint32_t c = a;
        while (c > lo && (key[c - 1] > k || (key[c - 1] == k && val[c - 1] > v))) {
            key[c] = key[c - 1];
            val[c] = val[c - 1];
            --c;
        }
        key[c] = k;
        val[c] = v;
    }
}

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

}  // namespace

void launch_keep_scan(Plan& p, hipStream_t st) {
    scan_keep_u32(p.keep, p.n_docs, p.kept_pos, p.scan, st);
    const uint64_t blocks = std::min<uint64_t>((p.n_docs + 255) / 256, 1024);
    const uint32_t lds = p.G <= LDS_GROUPS ? 1u : 0u;
    hipLaunchKernelGGL(k_compact_keys, dim3((uint32_t)blocks), dim3(256), lds ? sizeof(uint32_t) * p.G : 0, st, p,
                       p.key[0], p.val[0], p.hist, lds);
    DP_HIP(hipGetLastError());
}

// Sort of n (key64, val) pairs by (group[val], key64, val) into buffer 1 (the
// input is buffer 0); returns 1.  group values are < G; keys' high 32 bits
// uniform.  Launches are sized by the bucket bound n/2 + G + 1 (a group of
// n_g > 4 elements takes 2^b < n_g/2 buckets), so nothing is read back.
// counted: the group counts are in ws already and the bucket counts zeroed
// (the plan's sort: zeroed when the plan starts, counted by the compaction).
uint32_t sort_pairs(uint64_t* const key[2], uint32_t* const val[2], const uint32_t* group, uint64_t n, uint32_t G,
                    uint32_t* ws, const ScanWs& scan, uint32_t test_opts, bool counted, hipStream_t st) {
    if (n == 0) return 0;
    const uint64_t NB = n / 2 + G + 1;  // bucket bound
    uint32_t* gcount = ws;                 // [G]
    uint32_t* bcount = gcount + G;         // [NB], zeroed with gcount
    uint32_t* gbase = bcount + NB;         // [G + 1]
    uint32_t* boff = gbase + G + 1;        // [NB + 1]
    uint32_t* bucket = boff + NB + 1;      // [n]
    uint32_t* ticket = bucket + n;         // [n]
    const uint32_t blocks = (uint32_t)((n + 255) / 256);
    if (!counted) {
        launch_fill_u32(gcount, G + NB, 0u, st);
        const size_t glds = G <= LDS_GROUPS ? sizeof(uint32_t) * G : 0;
        hipLaunchKernelGGL(k_group_count, dim3(std::min<uint32_t>(blocks, 1024)), dim3(256), glds, st, val[0], group,
                           n, G, gcount);
    }
    if (G <= BASE_LDS_GROUPS) {
        hipLaunchKernelGGL(k_bucket_count<true>, dim3(blocks), dim3(256), 0, st, key[0], val[0], group, n, G,
                           (const uint32_t*)gcount, (const uint32_t*)nullptr, bcount, bucket, ticket);
    } else {
        hipLaunchKernelGGL(k_bucket_base, dim3(1), dim3(1024), 0, st, (const uint32_t*)gcount, G, gbase);
        hipLaunchKernelGGL(k_bucket_count<false>, dim3(blocks), dim3(256), 0, st, key[0], val[0], group, n, G,
                           (const uint32_t*)gcount, (const uint32_t*)gbase, bcount, bucket, ticket);
    }
    scan_u32(bcount, NB, boff, scan, st);
    hipLaunchKernelGGL(k_bucket_scatter, dim3(blocks), dim3(256), 0, st, key[0], val[0], n, (const uint32_t*)bucket,
                       (const uint32_t*)ticket, (const uint32_t*)boff, key[1], val[1]);
    hipLaunchKernelGGL(k_bucket_sort, dim3((uint32_t)((NB + 255) / 256)), dim3(256), 0, st, key[1], val[1],
                       (const uint32_t*)boff, NB, (test_opts & TEST_SORT_INSERTION) ? 1u : 0u);
    DP_HIP(hipGetLastError());
    return 1;
}

// requires p.n_kept (host) to be set
void launch_sort(Plan& p, hipStream_t st) {
    p.sort_buf = sort_pairs(p.key, p.val, p.group, p.n_kept, p.G, p.hist, p.scan, p.test_opts, true, st);
}

// requires perm_start (device) for the cycle; total = U·B
void launch_read_order(Plan& p, uint32_t cycle, uint64_t total, hipStream_t st) {
    if (total == 0) return;
    const uint32_t blocks = (uint32_t)((total + 255) / 256);
    hipLaunchKernelGGL(k_window_keys, dim3(blocks), dim3(256), 0, st, p, cycle, total);
    DP_HIP(hipGetLastError());
    const uint32_t buf = sort_pairs(p.wkey, p.wval, p.wgroup, total, p.S, p.hist, p.scan, p.test_opts, false, st);
    hipLaunchKernelGGL(k_perm_out, dim3(blocks), dim3(256), 0, st, p, (const uint32_t*)p.wval[buf], total);
    DP_HIP(hipGetLastError());
}

// the words of sort_pairs's workspace that hold its group and bucket counts
uint64_t sort_count_words(uint64_t n, uint64_t G) { return G + (n / 2 + G + 1); }

// workspace of sort_pairs for n pairs in G groups, in uint32 words
uint64_t sort_hist_words(uint64_t n, uint64_t G) {
    const uint64_t NB = n / 2 + G + 1;
    return G + NB + (G + 1) + (NB + 1) + 2 * n + 1 + 16;
}

}  // namespace dp
