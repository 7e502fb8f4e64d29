// hash.hip — corpus validation, per-document content hash and hold-out
// decision, per-source statistics.
//
// NeuronSpark-Trainer README, Concepts: 1 % of each file's documents (5 % for
// one source) are held out by a hash of their text that is the same in every
// data line; each source applies its own rate to that hash.  The hash here is
// the NH pair sum with fixed position keys k_i = (i+1)·0x9E3779B1, summed mod
// 2^64 (order-free, so a wavefront reduction gives the exact value), then the
// SplitMix64 output function over S xor L·0x9E3779B97F4A7C15.  A document is
// held iff floor(h·10000/2^64) < bp of its source, kept iff not held and
// non-empty.
#include "dp_common.h"

namespace dp {
namespace {

enum : uint32_t {
    ERR_OFFSETS = 1u,      // offsets decrease
    ERR_DOC_LEN = 2u,      // a document of 2^32 tokens or more
    ERR_SOURCE = 4u,       // source id out of range
    ERR_STRATUM = 8u,      // stratum id out of range for its source
    ERR_TOKENS = 16u,      // last offset beyond n_tokens
};

__global__ __launch_bounds__(256) void k_validate(Plan p) {
    const uint64_t d = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (d >= p.n_docs) return;
    uint32_t err = 0;
    const uint64_t o0 = p.offsets[d], o1 = p.offsets[d + 1];
    if (o1 < o0) err |= ERR_OFFSETS;
    else if (o1 - o0 > 0xFFFFFFFFull) err |= ERR_DOC_LEN;
    const uint32_t s = p.source[d];
    if (s >= p.S) {
        err |= ERR_SOURCE;
    } else {
        const uint32_t k = p.stratum ? p.stratum[d] : 0u;
        if (k >= p.n_strata[s]) err |= ERR_STRATUM;
        else p.group[d] = p.gbase[s] + k;
    }
    if (d == p.n_docs - 1 && o1 > p.n_tokens) err |= ERR_TOKENS;
    if (err) atomicOr(p.err, err);
}

// four tokens starting at a 4-byte aligned address: one global_load_dwordx4
// (multi-dword global loads need dword alignment only)
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

__device__ inline uint64_t quad_terms(const uint32_t* t, uint64_t base, uint64_t L) {
    uint32_t t0, t1 = 0, t2 = 0, t3 = 0;
    if (base + 4 <= L) {
        const u32x4a4 v = *reinterpret_cast<const u32x4a4*>(t + base);
        t0 = v.x; t1 = v.y; t2 = v.z; t3 = v.w;
    } else {
        t0 = t[base];
        if (base + 1 < L) t1 = t[base + 1];
        if (base + 2 < L) t2 = t[base + 2];
    }
    const uint32_t k0 = (uint32_t)(base + 1) * PHI32;
    const uint32_t k1 = k0 + PHI32, k2 = k1 + PHI32, k3 = k2 + PHI32;
    uint64_t S = (uint64_t)(t0 + k0) * (uint64_t)(t1 + k1);
    if (base + 2 < L) S += (uint64_t)(t2 + k2) * (uint64_t)(t3 + k3);
    return S;
}

// One wavefront per document (grid-stride).  Lane l takes the 4-token groups
// at document-relative indices 4l, 4l+256, …, i.e. two whole pairs each; an
// odd last token pairs with the virtual token 0 and its key.  Two groups per
// lane are loaded before either is used.
__global__ __launch_bounds__(256) void k_hash(Plan p, uint32_t lds_bins) {
    extern __shared__ unsigned long long bins[];  // [4][S] when lds_bins
    if (lds_bins) {
        for (uint32_t i = threadIdx.x; i < 4 * p.S; i += blockDim.x) bins[i] = 0;
        __syncthreads();
    }
    const uint32_t lane = lane_id();
    const uint64_t w0 = (uint64_t)__builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE);
    const uint64_t nw = (uint64_t)gridDim.x * (blockDim.x / WAVE);
    for (uint64_t d = w0; d < p.n_docs; d += nw) {
        const uint64_t o = p.offsets[d];
        const uint64_t L = p.offsets[d + 1] - o;
        const uint32_t* t = p.tokens + o;
        uint64_t S = 0;
        uint64_t base = 4ull * lane;
        for (; base + 4ull * WAVE < L; base += 8ull * WAVE) {
            const uint64_t s0 = quad_terms(t, base, L);
            const uint64_t s1 = quad_terms(t, base + 4ull * WAVE, L);
            S += s0 + s1;
        }
        if (base < L) S += quad_terms(t, base, L);
        S = wave_sum_u64(S);
        if (lane == 0) {
            const uint64_t h = mix64(S ^ (L * PHI64));
            const uint32_t s = p.source[d];
            const bool held = __umul64hi(h, 10000ull) < (uint64_t)p.bp[s];
            const bool keep = !held && L > 0;
            p.hash[d] = h;
            p.keep[d] = keep ? 1 : 0;
            if (held || keep) {
                const uint32_t slot = (held ? 2u : 0u) * p.S + s;
                if (lds_bins) {
                    atomicAdd(&bins[slot], 1ull);
                    atomicAdd(&bins[slot + p.S], (unsigned long long)L);
                } else {
                    atomicAdd((unsigned long long*)&p.stats[slot], 1ull);
                    atomicAdd((unsigned long long*)&p.stats[slot + p.S], (unsigned long long)L);
                }
            }
        }
    }
    if (lds_bins) {
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < 4 * p.S; i += blockDim.x)
            if (bins[i]) atomicAdd((unsigned long long*)&p.stats[i], bins[i]);
    }
}

}  // namespace

void launch_validate(const Plan& p, hipStream_t st) {
    const uint64_t blocks = (p.n_docs + 255) / 256;
    hipLaunchKernelGGL(k_validate, dim3((uint32_t)blocks), dim3(256), 0, st, p);
    DP_HIP(hipGetLastError());
}

void launch_hash(const Plan& p, hipStream_t st) {
    const uint32_t lds_bins = p.S <= 256 ? 1u : 0u;
    const size_t lds = lds_bins ? 4ull * p.S * sizeof(uint64_t) : 0;
    uint64_t blocks = (p.n_docs + 3) / 4;
    if (blocks > 8192) blocks = 8192;  // more blocks than resident slots: finished slots take new blocks
    hipLaunchKernelGGL(k_hash, dim3((uint32_t)blocks), dim3(256), lds, st, p, lds_bins);
    DP_HIP(hipGetLastError());
}

}  // namespace dp
