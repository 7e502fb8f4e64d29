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
#include <algorithm>

#include "dp_common.h"

namespace dp {
namespace {

enum : uint32_t {
    ERR_OFFSETS = 1u,      // offsets decrease
    ERR_DOC_LEN = 2u,      // a document of 2^32 tokens or more
    ERR_SOURCE = 4u,       // source id out of range
    ERR_STRATUM = 8u,      // stratum id out of range for its source
    ERR_TOKENS = 16u,      // last offset beyond n_tokens
    ERR_SEGMENT = 32u,     // arrival id out of range
};

constexpr uint32_t TPT = 16;         // contiguous tokens per thread of the hash
constexpr uint32_t HT = 256 * TPT;   // tokens per tile (one 256-thread block)

// One thread per document: the corpus checks, and two preparations of the
// hash (the validation visits every document anyway): the document's NH sum
// S[d] = 0, and the tile table first[t] = d for every tile whose first token
// base + t·HT lies in the document (each token belongs to one non-empty
// document, so every tile below ntiles gets exactly one writer; the last
// document also writes the sentinel first[ntiles] = D − 1).  A document whose
// own offsets are invalid writes no table entry, and entries stay below
// n_first, so an invalid corpus writes nothing out of place; the hash kernels
// then return at once on the error flag.
__global__ __launch_bounds__(256) void k_validate(Plan p, uint64_t* S, uint32_t* first, uint64_t n_first) {
    const uint64_t d = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (d >= p.n_docs) return;
    uint32_t err = 0;
    const uint64_t o0 = p.offsets[d], o1 = p.offsets[d + 1];
    S[d] = 0;
    if (o1 < o0) err |= ERR_OFFSETS;
    else if (o1 - o0 > 0xFFFFFFFFull) err |= ERR_DOC_LEN;
    const uint64_t base = p.offsets[0];
    if (!err && o1 > o0 && o0 >= base && o1 <= p.n_tokens) {
        for (uint64_t t = (o0 - base + HT - 1) / HT; t <= (o1 - 1 - base) / HT && t < n_first; ++t)
            first[t] = (uint32_t)d;
    }
    if (d == p.n_docs - 1 && o1 >= base) {
        const uint64_t ntiles = (o1 - base + HT - 1) / HT;
        if (ntiles < n_first) first[ntiles] = (uint32_t)d;
    }
    const uint32_t s = p.source[d];
    const uint32_t g = p.n_seg > 1 ? p.segment[d] : 0u;
    if (s >= p.S) {
        err |= ERR_SOURCE;
    } else if (g >= p.n_seg) {
        err |= ERR_SEGMENT;
    } else {
        const uint32_t k = p.stratum ? p.stratum[d] : 0u;
        if (k >= p.n_strata[s]) err |= ERR_STRATUM;
        else p.group[d] = p.gbase[s * p.n_seg + g] + k;  // groups (stream, arrival, stratum)
    }
    if (d == p.n_docs - 1 && o1 > p.n_tokens) err |= ERR_TOKENS;
    if (err) atomicOr(p.err, err);
}

// ------------------------------------------------------------------ flat hash
// The tokens of all documents form one contiguous range [off[0], off[D]).  It
// is cut into tiles of HT tokens; a thread takes TPT contiguous tokens, so the
// whole corpus streams through once, coalesced and balanced whatever the
// document lengths.  A token at document-relative index r (even) adds the NH
// term (t_r + k_r)·(t_{r+1} + k_{r+1}) to its document's sum, with t_L = 0 for
// an odd length L.  Per-document partial sums are combined inside a wavefront
// by a segmented scan (documents are in token order) and added to S[d] with one
// 64-bit atomic per document and wavefront: integer addition is order-free, so
// the sum is exact.  k_hash_final then mixes and decides the hold-out.
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

__device__ inline uint64_t pair_term(uint32_t a, uint32_t b, uint64_t r) {
    const uint32_t k0 = (uint32_t)(r + 1) * PHI32;
    return (uint64_t)(a + k0) * (uint64_t)(b + k0 + PHI32);
}

// The document offsets a tile needs are staged in LDS once per tile, so no
// thread waits on a dependent global load to find its documents (tiles with
// more than OCAP documents read them from global memory instead).
constexpr uint32_t OCAP = 1024;

struct Offs {
    const uint64_t* g;   // global offsets
    const uint64_t* l;   // LDS copy of offsets[d0 .. d0 + n)
    uint64_t d0;
    bool staged;
    __device__ inline uint64_t operator[](uint64_t d) const { return staged ? l[d - d0] : g[d]; }
};

// Loads the TPT + 1 tokens from t0 (the last one is the pair partner of the
// thread's last token), all in bounds: callers pass t0 + TPT + 1 <= end.
// (Non-temporal loads measured 1.6x slower here.)
__device__ __forceinline__ void load_tokens(const uint32_t* tokens, uint64_t t0, uint32_t (&x)[TPT + 1]) {
#pragma unroll
    for (uint32_t q = 0; q < TPT / 4; ++q) {
        const u32x4a4 v = *reinterpret_cast<const u32x4a4*>(tokens + t0 + 4 * q);
        x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
    }
    x[TPT] = tokens[t0 + TPT];
}

// A tile's documents [lo, hi] (from the tile table) and this thread's entry of
// their offsets, offsets[lo + threadIdx.x] (loaded ahead of the tile, so the
// staging below waits on no global load; entries past the first 256 are read
// at staging time).
struct TileMeta {
    uint64_t lo, hi, o;
};

__device__ __forceinline__ void meta_first(const uint32_t* first, uint64_t tile, TileMeta& m) {
    m.lo = first[tile];
    m.hi = first[tile + 1];
}

__device__ __forceinline__ void meta_offset(const Plan& p, TileMeta& m) {
    m.o = threadIdx.x < m.hi - m.lo + 2 ? p.offsets[m.lo + threadIdx.x] : 0;
}

// One tile: the tile's document offsets into LDS, each thread's documents and
// NH terms, and the per-document sums into S (see above).  x holds the
// thread's tokens from t0 (zeros past end).  FULL: every thread's TPT + 1
// tokens lie below end.
//
// A wavefront whose tokens and last partner lie in one document (most of them:
// a wavefront spans 1,025 tokens, documents average about 1,200) takes a
// branch-free path: the thread's pairs start at the positions whose offset in
// the document is even, TPT/2 products accumulated with 32x32→64 multiply-adds,
// then one wavefront sum and one atomic.  Other wavefronts walk the thread's
// positions with document offsets kept in 32 bits: only r mod 2^32 enters a
// key, and a thread's positions are within TPT + 1 of its document's end.
template <bool FULL>
__device__ __forceinline__ void hash_tile(const Plan& p, uint64_t base, uint64_t end, uint64_t tile,
                                          const uint32_t (&x)[TPT + 1], const TileMeta& m, uint64_t* s_off,
                                          uint64_t* S) {
    const uint32_t lane = lane_id();
    const uint64_t t0 = base + tile * HT + (uint64_t)TPT * threadIdx.x;  // this thread's first token
    const uint64_t d_lo = m.lo, d_hi = m.hi;  // documents of the tile
    const uint64_t n_off = d_hi - d_lo + 2;
    Offs off{p.offsets, s_off, d_lo, n_off <= OCAP + 1};
    __syncthreads();  // the previous tile's readers are done with s_off
    if (off.staged) {
        if (threadIdx.x < n_off) s_off[threadIdx.x] = m.o;
        for (uint64_t i = threadIdx.x + blockDim.x; i < n_off; i += blockDim.x) s_off[i] = p.offsets[d_lo + i];
    }
    __syncthreads();
    const bool active = FULL || t0 < end;
    uint32_t cur = 0;
    uint64_t ob = 0, nb = 0;
    if (active) {
        // document of t0: search between the tile's first document and the next tile's
        uint64_t lo = d_lo, hi = d_hi + 1;  // d in [lo, hi)
        while (hi - lo > 1) {
            const uint64_t mid = (lo + hi) >> 1;
            if (off[mid] <= t0) lo = mid;
            else hi = mid;
        }
        cur = (uint32_t)lo;
        ob = off[cur];
        nb = off[cur + 1];
    }
    if (__all(active && t0 + TPT < nb)) {
        // one document under the whole wavefront: offsets r = rb + j, pairs at
        // j = par, par + 2, ..., keys k = (r + 1)·φ32 and k + φ32
        const uint32_t rb = (uint32_t)(t0 - ob);
        const uint32_t par = rb & 1u;
        const uint32_t kp = (rb + 1u + par) * PHI32;
        uint64_t acc = 0;
#pragma unroll
        for (uint32_t i = 0; i < TPT / 2; ++i) {
            const uint32_t a = par ? x[2 * i + 1] : x[2 * i];
            const uint32_t b = par ? x[2 * i + 2] : x[2 * i + 1];
            const uint32_t k0 = kp + 2u * i * PHI32;
            acc += (uint64_t)(a + k0) * (uint64_t)(b + k0 + PHI32);
        }
        acc = wave_sum_u64(acc);
        if (lane == 0) atomicAdd((unsigned long long*)&S[cur], (unsigned long long)acc);
        return;
    }
    uint32_t fd = 0xFFFFFFFFu, ld = 0xFFFFFFFFu;
    uint64_t v1 = 0, v2 = 0;
    if (active) {
        fd = cur;
        // rem: positions from t0 before the document's end, capped at TPT + 1;
        // kb: the key of offset rb, (rb + 1)·φ32, so offset rb + j has kb + j·φ32
        uint32_t rem = (uint32_t)std::min<uint64_t>(nb - t0, TPT + 1);
        uint32_t rb = (uint32_t)(t0 - ob);
        uint32_t kb = (rb + 1u) * PHI32;
        bool e0 = (rb & 1u) == 0;  // offset rb + j is even iff e0 == (j even)
        const uint32_t n_in = FULL ? TPT : (uint32_t)std::min<uint64_t>(end - t0, TPT);
        uint64_t acc = 0;
#pragma unroll
        for (uint32_t j = 0; j < TPT; ++j) {
            if (FULL || j < n_in) {
                if (j >= rem) {  // the next document starts: flush the finished one
                    if (cur == fd) v1 = acc;
                    else atomicAdd((unsigned long long*)&S[cur], (unsigned long long)acc);
                    acc = 0;
                    do {
                        ++cur;
                        ob = nb;
                        nb = off[cur + 1];
                    } while (t0 + j >= nb);
                    rem = (uint32_t)std::min<uint64_t>(nb - t0, TPT + 1);
                    rb = (uint32_t)(t0 - ob);  // the offset of t0, mod 2^32
                    kb = (rb + 1u) * PHI32;
                    e0 = (rb & 1u) == 0;
                }
                // a term at even offsets only: its first factor is zeroed at odd ones
                const uint32_t k0 = kb + j * PHI32;
                const uint32_t b = j + 1 < rem ? x[j + 1] : 0u;
                const uint32_t a = (e0 == ((j & 1u) == 0)) ? x[j] + k0 : 0u;
                acc += (uint64_t)a * (uint64_t)(b + k0 + PHI32);
            }
        }
        if (cur == fd) v1 = acc;
        else {
            ld = cur;
            v2 = acc;
        }
    }
    // the last document's part joins the next lane's first document when they match
    const uint32_t fd_next = __shfl_down(fd, 1, WAVE);
    if (ld != 0xFFFFFFFFu && (lane == WAVE - 1 || fd_next != ld))
        atomicAdd((unsigned long long*)&S[ld], (unsigned long long)v2);
    const uint32_t ld_prev = __shfl_up(ld, 1, WAVE);
    const uint64_t v2_prev = __shfl_up(v2, 1, WAVE);
    if (lane > 0 && ld_prev != 0xFFFFFFFFu && ld_prev == fd) v1 += v2_prev;
    // segmented inclusive scan of v1 by fd (fd is nondecreasing across lanes)
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const uint64_t y = __shfl_up(v1, o, WAVE);
        const uint32_t fy = __shfl_up(fd, o, WAVE);
        if (lane >= (uint32_t)o && fy == fd) v1 += y;
    }
    if (fd != 0xFFFFFFFFu && (lane == WAVE - 1 || fd_next != fd))
        atomicAdd((unsigned long long*)&S[fd], (unsigned long long)v1);
}

// Tiles [0, nfast) have every thread's TPT + 1 tokens inside [base, end):
// they run two at a time in a software pipeline whose loads are issued (at a
// clamped tile, unconditionally) before the current tile is hashed: the next
// tile's tokens and offset entries, and the tile table two tiles ahead.  A
// tile's hashing then waits on no global load.  The last tiles load element
// by element with bounds checks.
__global__ __launch_bounds__(256) void k_hash_flat(Plan p, const uint32_t* first, uint64_t* S) {
    if (*p.err) return;  // an invalid corpus: nothing reads its offsets
    const uint64_t base = p.offsets[0], end = p.offsets[p.n_docs];
    if (end == base) return;
    const uint64_t ntiles = (end - base + HT - 1) / HT;
    const uint64_t nfast = (end - base - 1) / HT;  // tiles whose every thread reads TPT + 1 tokens below end
    __shared__ uint64_t s_off[OCAP + 1];
    const uint32_t* tok = p.tokens;
    const uint64_t step = gridDim.x;
    uint64_t ta = blockIdx.x;
    if (ta < nfast) {
        uint32_t xa[TPT + 1], xb[TPT + 1];
        TileMeta ma, mb, mc;
        meta_first(first, ta, ma);
        meta_offset(p, ma);
        load_tokens(tok, base + ta * HT + (uint64_t)TPT * threadIdx.x, xa);
        uint64_t tb = ta + step, cb = tb < nfast ? tb : ta;  // cb: a tile below nfast to load from
        meta_first(first, cb, mb);
        while (true) {
            // ta ready (xa, ma); tb's table entries ready (mb)
            load_tokens(tok, base + cb * HT + (uint64_t)TPT * threadIdx.x, xb);
            meta_offset(p, mb);
            const uint64_t tc = tb + step, cc = tc < nfast ? tc : cb;
            meta_first(first, cc, mc);
            hash_tile<true>(p, base, end, ta, xa, ma, s_off, S);
            if (tb >= nfast) break;
            // tb ready (xb, mb); tc's table entries ready (mc)
            load_tokens(tok, base + cc * HT + (uint64_t)TPT * threadIdx.x, xa);
            ma = mc;
            meta_offset(p, ma);
            const uint64_t td = tc + step, cd = td < nfast ? td : cc;
            meta_first(first, cd, mc);
            hash_tile<true>(p, base, end, tb, xb, mb, s_off, S);
            if (tc >= nfast) break;
            ta = tc;
            tb = td;
            cb = cd;
            mb = mc;
        }
    }
    for (uint64_t tile = nfast + blockIdx.x; tile < ntiles; tile += step) {
        const uint64_t t0 = base + tile * HT + (uint64_t)TPT * threadIdx.x;
        uint32_t x[TPT + 1];
#pragma unroll
        for (uint32_t j = 0; j <= TPT; ++j) x[j] = (t0 + j < end) ? tok[t0 + j] : 0u;
        TileMeta m;
        meta_first(first, tile, m);
        meta_offset(p, m);
        hash_tile<false>(p, base, end, tile, x, m, s_off, S);
    }
}

// h = mix64(S xor L·φ64); held iff floor(h·10000/2^64) < bp; kept iff not held
// and non-empty (with the held-out stream: iff held and non-empty); per-source
// statistics in LDS, one atomic per block and bin.
__global__ __launch_bounds__(256) void k_hash_final(Plan p, const uint64_t* S, uint32_t lds_bins) {
    if (*p.err) return;  // an invalid corpus: source ids may be out of range
    extern __shared__ unsigned long long bins[];  // [4][S] when lds_bins
    if (lds_bins) {
        for (uint32_t i = threadIdx.x; i < 4 * p.S; i += blockDim.x) bins[i] = 0;
        __syncthreads();
    }
    for (uint64_t d = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; d < p.n_docs;
         d += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t L = p.offsets[d + 1] - p.offsets[d];
        const uint64_t h = mix64(S[d] ^ (L * PHI64));
        const uint32_t s = p.source[d];
        const bool held = __umul64hi(h, 10000ull) < (uint64_t)p.bp[s];
        const bool keep = (p.heldout ? held : !held) && L > 0;  // the stream's documents
        p.hash[d] = h;
        p.keep[d] = keep ? 1 : 0;
        for (uint32_t b = 0; b < 2; ++b) {  // bins 0: the stream's documents, 2: held out by the hash
            if (!(b == 0 ? keep : held)) continue;
            const uint32_t slot = 2u * b * p.S + s;
            if (lds_bins) {
                atomicAdd(&bins[slot], 1ull);
                atomicAdd(&bins[slot + p.S], (unsigned long long)L);
            } else {
                atomicAdd((unsigned long long*)&p.stats[slot], 1ull);
                atomicAdd((unsigned long long*)&p.stats[slot + p.S], (unsigned long long)L);
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

void launch_validate(const Plan& p, uint64_t* S, uint32_t* first, hipStream_t st) {
    const uint64_t blocks = (p.n_docs + 255) / 256;
    hipLaunchKernelGGL(k_validate, dim3((uint32_t)blocks), dim3(256), 0, st, p, S, first,
                       hash_tile_count(p.n_tokens) + 2);
    DP_HIP(hipGetLastError());
}

// S: [n_docs] sums, zeroed by the validation kernel; first: the tile table it
// wrote ([hash_tile_count(n_tokens) + 2]).  The span [offsets[0],
// offsets[n_docs]) is read on the device and the grid is sized by n_tokens, so
// nothing waits for the validation: after an invalid corpus the kernels return
// at once and the error is read with the kept count.
void launch_hash(const Plan& p, uint64_t* S, uint32_t* first, hipStream_t st) {
    const uint64_t ntiles = (p.n_tokens + HT - 1) / HT;  // a bound: the documents cover at most n_tokens
    if (ntiles)
        hipLaunchKernelGGL(k_hash_flat, dim3((uint32_t)std::min<uint64_t>(ntiles, 16384)), dim3(256), 0, st, p,
                           (const uint32_t*)first, S);
    const uint32_t lds_bins = p.S <= 256 ? 1u : 0u;
    const size_t lds = lds_bins ? 4ull * p.S * sizeof(uint64_t) : 0;
    hipLaunchKernelGGL(k_hash_final, dim3((uint32_t)std::min<uint64_t>((p.n_docs + 255) / 256, 1024)), dim3(256), lds,
                       st, p, (const uint64_t*)S, lds_bins);
    DP_HIP(hipGetLastError());
}

uint64_t hash_tile_count(uint64_t n_tokens) { return (n_tokens + HT - 1) / HT; }

}  // namespace dp
