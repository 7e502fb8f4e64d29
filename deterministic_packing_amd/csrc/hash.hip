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

constexpr uint32_t TPT = 16;          // contiguous tokens per lane of the hash
constexpr uint32_t WT = WAVE * TPT;   // tokens per wave-tile (one wavefront's share)

// One thread per document: the corpus checks, and preparations of later steps
// (the validation visits every document anyway): zero the plan's two sums
// (added to at the end of the plan), the document's NH sum S[d] = 0, and the
// hash's tile table first[t] = d for every wave-tile whose first
// token base + t·WT lies in the document (each token belongs to one non-empty
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
    if (d == 0) p.checks[0] = p.checks[1] = 0;  // the plan's two sums, added to at the end of the plan
    if (o1 < o0) err |= ERR_OFFSETS;
    else if (o1 - o0 > 0xFFFFFFFFull) err |= ERR_DOC_LEN;
    const uint64_t base = p.offsets[0];
    if (!err && o1 > o0 && o0 >= base && o1 <= p.n_tokens) {
        for (uint64_t t = (o0 - base + WT - 1) / WT; t <= (o1 - 1 - base) / WT && t < n_first; ++t)
            first[t] = (uint32_t)d;
    }
    if (d == p.n_docs - 1 && o1 >= base) {
        const uint64_t ntiles = (o1 - base + WT - 1) / WT;
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
// The tokens of all documents form one contiguous range [off[0], off[D)),
// cut into wave-tiles of WT tokens; lane l of a wavefront takes the TPT
// contiguous tokens from the tile start + TPT·l, so the corpus streams through
// once, coalesced and balanced whatever the document lengths.  Every
// wavefront works on its own, with neither LDS nor barriers: a tile's
// documents come from the tile table, and lane k holds the offset of the
// tile's k-th document.  A token at document-relative index r (even) adds the
// NH term (t_r + k_r)·(t_{r+1} + k_{r+1}) to its document's sum, with t_L = 0
// for an odd length L.  Per-document partial sums are combined by a segmented
// scan across the wavefront (documents are in token order) and added to S[d]
// with one 64-bit atomic per document and tile: integer addition is
// order-free, so the sum is exact.  k_hash_final then mixes and decides the
// hold-out.
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

// Loads the TPT + 1 tokens from t0 (the last one is the pair partner of the
// lane's last token), all in bounds: callers pass t0 + TPT + 1 <= end.
// (Non-temporal loads measured 1.6x slower here.)
__device__ __forceinline__ void load_tokens(const uint32_t* tokens, uint64_t t0, uint32_t (&x)[TPT + 1]) {
#pragma unroll
    for (uint32_t q = 0; q < TPT / 4; ++q) {
        const u32x4a4 v = *reinterpret_cast<const u32x4a4*>(tokens + t0 + 4 * q);
        x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
    }
    x[TPT] = tokens[t0 + TPT];
}

// One step of an inclusive scan of v segmented by the key f (nondecreasing
// across lanes): the source lane's partial is added when its key is the same.
template <int CTRL, int ROWS>
__device__ __forceinline__ void seg_step(uint64_t& v, uint32_t f) {
    const uint32_t fy = dpp32<CTRL, ROWS>(0xFFFFFFFFu, f);
    const uint64_t y = dpp64<CTRL, ROWS>(0, v);
    if (fy == f) v += y;
}

__device__ __forceinline__ void seg_scan(uint64_t& v, uint32_t f) {
    seg_step<DPP_ROW_SHR1, 0xF>(v, f);
    seg_step<DPP_ROW_SHR2, 0xF>(v, f);
    seg_step<DPP_ROW_SHR4, 0xF>(v, f);
    seg_step<DPP_ROW_SHR8, 0xF>(v, f);
    seg_step<DPP_BCAST15, 0xA>(v, f);
    seg_step<DPP_BCAST31, 0xC>(v, f);
}

constexpr uint32_t NO_END = 0xFFFFFFFFu;  // no further document start within reach of the lane

// What a wave-tile needs besides its tokens: the documents lo and hi holding
// its first token and the next tile's (tile table), off[lo], and lane k's
// offset off[lo + k] for k ≤ hi − lo (clamped to off[D]), which serves tiles
// of hi − lo < WAVE.
// Every load is a vector load (lane 0 and 1 read the two table entries; lane
// 0's offset is off[lo]), counted in order with the token loads, so waiting
// for one tile's entries never waits for loads issued after them.
struct TileDocs {
    uint64_t lo, hi, olo, o;
    uint32_t tv;  // lane 0: first[t], lane 1: first[t + 1]
};

__device__ __forceinline__ void tile_table(const uint32_t* first, uint64_t t, TileDocs& m) {
    m.tv = first[t + std::min<uint32_t>(lane_id(), 1u)];
}

__device__ __forceinline__ void tile_offsets(const Plan& p, TileDocs& m) {
    m.lo = (uint32_t)__builtin_amdgcn_readlane((int)m.tv, 0);
    m.hi = (uint32_t)__builtin_amdgcn_readlane((int)m.tv, 1);
    // only the lanes of the tile's documents load (a tile inside one document: lane 0 alone)
    m.o = lane_id() <= m.hi - m.lo ? p.offsets[std::min<uint64_t>(m.lo + lane_id(), p.n_docs)] : 0;
}

__device__ __forceinline__ void tile_ready(TileDocs& m) { m.olo = readlane64(m.o, 0); }

// One wave-tile [wb, wb + WT).  x: the lane's tokens from t0 = wb + TPT·lane
// (zeros at and past end).  FULL: every lane's TPT + 1 tokens lie below end.
//
// A tile whose tokens and last partner lie in one document (lo == hi) takes a
// branch-free path: the pairs start where the document offset is even (the
// same parity in every lane), TPT/2 products accumulated with 32x32→64
// multiply-adds, one wavefront sum and one atomic.  In other tiles each lane
// finds its document and the next two document starts from the offsets the
// lanes hold (or, past WAVE documents in the tile, by a binary search), then
// walks its positions with document offsets kept in 32 bits: only r mod 2^32
// enters a key, and a lane's positions are within TPT + 1 of its document's end.
template <bool FULL>
__device__ __forceinline__ void hash_wave_tile(const Plan& p, uint64_t end, uint64_t wb,
                                               const uint32_t (&x)[TPT + 1], const TileDocs& m, uint64_t* S) {
    const uint32_t lane = lane_id();
    const uint64_t t0 = wb + (uint64_t)TPT * lane;
    if (FULL && m.lo == m.hi) {
        const uint32_t par = (uint32_t)(wb - m.olo) & 1u;  // parity of the document offset of t0
        const uint32_t kp = ((uint32_t)(t0 - m.olo) + 1u + par) * PHI32;
        uint64_t acc = 0;
#pragma unroll
        for (uint32_t i = 0; i < TPT / 2; ++i) {
            const uint32_t a = par ? x[2 * i + 1] : x[2 * i];
            const uint32_t b = par ? x[2 * i + 2] : x[2 * i + 1];
            const uint32_t k0 = kp + 2u * i * PHI32;
            acc += (uint64_t)(a + k0) * (uint64_t)(b + k0 + PHI32);
        }
        acc = wave_incl_u64(acc);
        if (lane == WAVE - 1) atomicAdd((unsigned long long*)&S[m.lo], (unsigned long long)acc);
        return;
    }
    const bool active = FULL || t0 < end;
    // the lane's document cur, the offset rb of t0 in it (mod 2^32), and the
    // distances dn, dn2 from t0 to the next two document starts (NO_END: none
    // in the tile, or farther than any position of the lane)
    uint32_t cur = (uint32_t)m.lo, rb = (uint32_t)(t0 - m.olo), dn = NO_END, dn2 = NO_END;
    if (m.hi - m.lo < WAVE) {
        // positions relative to wb: the tile's later documents start in (0, WT]
        const uint32_t tr = TPT * lane;
        uint32_t kc = 0, obr = 0, nbr = NO_END, nb2r = NO_END;
        for (uint32_t k = (uint32_t)(m.hi - m.lo); k >= 1; --k) {
            const uint32_t sr = (uint32_t)(readlane64(m.o, k) - wb);
            if (sr > tr) {
                nb2r = nbr;
                nbr = sr;
            } else if (kc == 0) {
                kc = k;
                obr = sr;
            }
        }
        if (kc) {
            cur += kc;
            rb = tr - obr;
        }
        if (nbr != NO_END) dn = nbr - tr;
        if (nb2r != NO_END) dn2 = nb2r - tr;
    } else if (active) {
        uint64_t lo = m.lo, hi = m.hi + 1;  // cur in [lo, hi)
        while (hi - lo > 1) {
            const uint64_t mid = (lo + hi) >> 1;
            if (p.offsets[mid] <= t0) lo = mid;
            else hi = mid;
        }
        cur = (uint32_t)lo;
        rb = (uint32_t)(t0 - p.offsets[lo]);
        if (lo + 1 <= m.hi) dn = (uint32_t)std::min<uint64_t>(p.offsets[lo + 1] - t0, NO_END);
        if (lo + 2 <= m.hi) dn2 = (uint32_t)std::min<uint64_t>(p.offsets[lo + 2] - t0, NO_END);
    }
    uint32_t fd = 0xFFFFFFFFu, ld = 0xFFFFFFFFu;
    uint64_t v1 = 0, v2 = 0;
    if (active) {
        fd = cur;
        // rem: positions from t0 before the document's end, capped at TPT + 1;
        // kb: the key of offset rb, (rb + 1)·φ32, so offset rb + j has kb + j·φ32
        uint32_t rem = std::min<uint32_t>(dn, TPT + 1);
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
                    do {  // t0 lies dn before the new document's start: its offset is −dn
                        ++cur;
                        rb = 0u - dn;
                        dn = dn2;
                        dn2 = cur + 2 <= m.hi ? (uint32_t)std::min<uint64_t>(p.offsets[cur + 2] - t0, NO_END) : NO_END;
                    } while (j >= dn);
                    rem = std::min<uint32_t>(dn, TPT + 1);
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
    // the lane's last document part joins the next lane's first document when
    // they are the same document; the rest is scanned by first document
    const uint32_t fd_next = dpp32<DPP_WAVE_SHL1, 0xF>(0xFFFFFFFFu, fd);
    const uint32_t ld_prev = dpp32<DPP_WAVE_SHR1, 0xF>(0xFFFFFFFFu, ld);
    const uint64_t v2_prev = dpp64<DPP_WAVE_SHR1, 0xF>(0, v2);
    if (ld != 0xFFFFFFFFu && fd_next != ld) atomicAdd((unsigned long long*)&S[ld], (unsigned long long)v2);
    if (ld_prev != 0xFFFFFFFFu && ld_prev == fd) v1 += v2_prev;
    seg_scan(v1, fd);
    if (fd != 0xFFFFFFFFu && fd_next != fd) atomicAdd((unsigned long long*)&S[fd], (unsigned long long)v1);
}

// Wave-tiles [0, nfast) have every lane's TPT + 1 tokens inside [base, end):
// a wavefront takes them two at a time in a software pipeline whose loads are
// issued (at a clamped tile, unconditionally) before the current tile is
// hashed: the next tile's tokens and offsets, and the tile table two tiles
// ahead.  The last tile loads element by element with bounds checks.
__global__ __launch_bounds__(256) void k_hash_flat(Plan p, const uint32_t* first, uint64_t* S) {
    if (*p.err) return;  // an invalid corpus: nothing reads its offsets
    const uint64_t base = p.offsets[0], end = p.offsets[p.n_docs];
    if (end == base) return;
    const uint64_t ntiles = (end - base + WT - 1) / WT;
    const uint64_t nfast = (end - base - 1) / WT;  // tiles whose every lane reads TPT + 1 tokens below end
    const uint32_t* tok = p.tokens;
    const uint64_t step = (uint64_t)gridDim.x * (blockDim.x / WAVE);
    const uint64_t wave0 = (uint64_t)blockIdx.x * (blockDim.x / WAVE) +
                           (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const uint32_t lane_t = TPT * lane_id();
    uint64_t ta = wave0;
    if (ta < nfast) {
        uint32_t xa[TPT + 1], xb[TPT + 1];
        TileDocs ma, mb, mc;
        tile_table(first, ta, ma);
        tile_offsets(p, ma);
        load_tokens(tok, base + ta * WT + lane_t, xa);
        uint64_t tb = ta + step, cb = tb < nfast ? tb : ta;  // cb: a tile below nfast to load from
        tile_table(first, cb, mb);
        while (true) {
            // ta ready (xa, ma); tb's table entries ready (mb)
            load_tokens(tok, base + cb * WT + lane_t, xb);
            tile_offsets(p, mb);
            const uint64_t tc = tb + step, cc = tc < nfast ? tc : cb;
            tile_table(first, cc, mc);
            tile_ready(ma);
            hash_wave_tile<true>(p, end, base + ta * WT, xa, ma, S);
            if (tb >= nfast) break;
            // tb ready (xb, mb); tc's table entries ready (mc)
            load_tokens(tok, base + cc * WT + lane_t, xa);
            ma = mc;
            tile_offsets(p, ma);
            const uint64_t td = tc + step, cd = td < nfast ? td : cc;
            tile_table(first, cd, mc);
            tile_ready(mb);
            hash_wave_tile<true>(p, end, base + tb * WT, xb, mb, S);
            if (tc >= nfast) break;
            ta = tc;
            tb = td;
            cb = cd;
            mb = mc;
        }
    }
    for (uint64_t t = nfast + wave0; t < ntiles; t += step) {
        const uint64_t t0 = base + t * WT + lane_t;
        uint32_t x[TPT + 1];
#pragma unroll
        for (uint32_t j = 0; j <= TPT; ++j) x[j] = (t0 + j < end) ? tok[t0 + j] : 0u;
        TileDocs m;
        tile_table(first, t, m);
        tile_offsets(p, m);
        tile_ready(m);
        hash_wave_tile<false>(p, end, base + t * WT, x, m, S);
    }
}

// h = mix64(S xor L·φ64); held iff floor(h·10000/2^64) < bp; kept iff not held
// and non-empty (with the held-out stream: iff held and non-empty); per-source
// statistics in LDS, one atomic per block and bin.  A wavefront takes FD
// groups of 64 consecutive documents per pass and issues all their loads
// before it computes any of them (the stores of one document would otherwise
// keep the next document's loads behind them).  A group whose documents share
// one source (documents usually come grouped by source) adds its counts and
// lengths with one atomic per bin; others, one per document.
constexpr uint32_t FD = 4;

__device__ __forceinline__ void add_bin(unsigned long long* bins, uint64_t* stats, uint32_t slot, uint64_t v,
                                        bool lds) {
    if (lds) atomicAdd(&bins[slot], (unsigned long long)v);
    else atomicAdd((unsigned long long*)&stats[slot], (unsigned long long)v);
}

__global__ __launch_bounds__(256) void k_hash_final(Plan p, const uint64_t* S, uint32_t lds_bins) {
    if (*p.err) return;  // an invalid corpus: source ids may be out of range
    extern __shared__ unsigned long long bins[];  // [4][S] when lds_bins, then bp [S] as u32
    uint32_t* s_bp = reinterpret_cast<uint32_t*>(bins + 4 * p.S);
    if (lds_bins) {
        for (uint32_t i = threadIdx.x; i < 4 * p.S; i += blockDim.x) bins[i] = 0;
        for (uint32_t i = threadIdx.x; i < p.S; i += blockDim.x) s_bp[i] = p.bp[i];
        __syncthreads();
    }
    const uint32_t lane = lane_id();
    const uint64_t per_wave = (uint64_t)FD * WAVE;
    const uint64_t stride = (uint64_t)gridDim.x * (blockDim.x / WAVE) * per_wave;
    for (uint64_t g0 = ((uint64_t)blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE) * per_wave; g0 < p.n_docs;
         g0 += stride) {
        uint64_t o0[FD], o1[FD], sum[FD];
        uint32_t src[FD];
#pragma unroll
        for (uint32_t k = 0; k < FD; ++k) {
            const uint64_t d = std::min<uint64_t>(g0 + k * WAVE + lane, p.n_docs - 1);  // clamped: loads stay in bounds
            o0[k] = p.offsets[d];
            o1[k] = p.offsets[d + 1];
            sum[k] = S[d];
            src[k] = p.source[d];
        }
#pragma unroll
        for (uint32_t k = 0; k < FD; ++k) {
            const uint64_t g = g0 + k * WAVE;
            if (g >= p.n_docs) break;  // uniform
            const uint64_t d = g + lane;
            const bool valid = d < p.n_docs;
            const uint64_t L = o1[k] - o0[k];
            const uint32_t s = src[k];
            const uint64_t h = mix64(sum[k] ^ (L * PHI64));
            const bool held = valid && __umul64hi(h, 10000ull) < (uint64_t)(lds_bins ? s_bp[s] : p.bp[s]);
            const bool keep = valid && (p.heldout ? held : !held) && L > 0;  // the stream's documents
            if (valid) {
                p.hash[d] = h;
                p.keep[d] = keep ? 1 : 0;
            }
            // bins 0: the stream's documents, 2: held out by the hash ([count, length] per source)
            const uint32_t s0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)s);  // lane 0 is valid
            if (__all(!valid || s == s0)) {
                const uint64_t kc = __popcll(__ballot(keep)), hc = __popcll(__ballot(held));
                const uint64_t kl = wave_incl_u64(keep ? L : 0), hl = wave_incl_u64(held ? L : 0);
                if (lane == WAVE - 1) {
                    if (kc) {
                        add_bin(bins, p.stats, s0, kc, lds_bins);
                        add_bin(bins, p.stats, p.S + s0, kl, lds_bins);
                    }
                    if (hc) {
                        add_bin(bins, p.stats, 2 * p.S + s0, hc, lds_bins);
                        add_bin(bins, p.stats, 3 * p.S + s0, hl, lds_bins);
                    }
                }
            } else {
                for (uint32_t b = 0; b < 2; ++b) {
                    if (!(b == 0 ? keep : held)) continue;
                    const uint32_t slot = 2u * b * p.S + s;
                    add_bin(bins, p.stats, slot, 1, lds_bins);
                    add_bin(bins, p.stats, slot + p.S, L, lds_bins);
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
    const uint64_t ntiles = (p.n_tokens + WT - 1) / WT;  // a bound: the documents cover at most n_tokens
    if (ntiles)
        hipLaunchKernelGGL(k_hash_flat, dim3((uint32_t)std::clamp<uint64_t>(ntiles / 32, 1, 65536)), dim3(256), 0, st,
                           p, (const uint32_t*)first, S);
    const uint32_t lds_bins = p.S <= 256 ? 1u : 0u;
    const size_t lds = lds_bins ? 4ull * p.S * sizeof(uint64_t) + p.S * sizeof(uint32_t) : 0;
    const uint64_t groups = (p.n_docs + FD * WAVE - 1) / (FD * WAVE);  // of FD·64 documents, one per wavefront
    hipLaunchKernelGGL(k_hash_final, dim3((uint32_t)std::clamp<uint64_t>((groups + 3) / 4, 1, 2048)), dim3(256), lds, st,
                       p, (const uint64_t*)S, lds_bins);
    DP_HIP(hipGetLastError());
}

uint64_t hash_tile_count(uint64_t n_tokens) { return (n_tokens + WT - 1) / WT; }

}  // namespace dp
