// plan.hip — strata merge, pieces, next-fit window cut, mixture slots and the
// plan's order checks.  Every step here computes its result as a closed-form
// rank or a function composition, so the output is independent of thread
// scheduling and equal to the sequential definition.
#include <algorithm>

#include "dp_common.h"

namespace dp {
namespace {

__device__ inline uint32_t upper_bound_u64(const uint64_t* a, uint32_t n, uint64_t x) {
    // first index i in [0, n) with a[i] > x (n if none)
    uint32_t lo = 0, hi = n;
    while (lo < hi) {
        const uint32_t mid = (lo + hi) >> 1;
        if (a[mid] <= x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// ------------------------------------------------------------------ A4 strata merge
// NeuronSpark-Trainer README, Concepts: every segment of a cycle holds each
// stratum of a source at its share of the source's tokens, cut at document
// ends, in proportion to the strata's sizes.  Sequential reading: repeatedly
// take the head of the stratum with the least consumed fraction a_k/A_k, ties
// to the lower stratum.  Each stratum's fractions increase strictly, so the
// result is the merge of the strata by (a/A, k) and the output position of
// element (k, j) is j plus, for every other stratum k', the number of its
// elements ordered before it — counted by binary search with exact 128-bit
// cross-multiplication.  The merged order's token prefix comes the same way:
// the element's stratum's tokens before it plus, for every other stratum, the
// tokens of the elements counted before it (and the units before its own).

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* a, uint64_t n, uint32_t v) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) a[i] = v;
}

// one block per range: 4-byte words, then the last bytes
__global__ __launch_bounds__(256) void k_xfer(XferList l) {
    const Xfer x = l.x[blockIdx.x];
    const uint64_t words = x.bytes / 4;
    const uint32_t* s = reinterpret_cast<const uint32_t*>(x.src);
    uint32_t* d = reinterpret_cast<uint32_t*>(x.dst);
    for (uint64_t i = threadIdx.x; i < words; i += blockDim.x) d[i] = s[i];
    for (uint64_t i = 4 * words + threadIdx.x; i < x.bytes; i += blockDim.x) x.dst[i] = x.src[i];
}

// group_start[g] for every group: the sorted documents come group by group,
// so the element where the group changes writes the start of its group and of
// the empty groups just before it (the first element from group 0 on, the last
// one the empty groups after it, up to group_start[G] = n).  Each entry has
// one writer.  Also clears the merged order (holes, which a correct merge
// never leaves, would then read document 0).
__global__ __launch_bounds__(256) void k_group_bounds(const uint32_t* val, const uint32_t* group, uint64_t n,
                                                      uint32_t G, uint32_t* gs, uint32_t* order) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    order[i] = 0;
    const uint32_t g = group[val[i]];
    const uint32_t from = i == 0 ? 0u : group[val[i - 1]] + 1;  // groups from .. g start here
    for (uint32_t x = from; x <= g && x < G; ++x) gs[x] = (uint32_t)i;
    if (i == n - 1)
        for (uint32_t x = g + 1; x <= G; ++x) gs[x] = (uint32_t)n;
}

// Number of elements of stratum k2 (documents [c0, c1) of the group order,
// prefix gpre) that come before an element of stratum k at consumed fraction
// a/A: a2/A2 < a/A, or equal and k2 < k; searched in [lo, hi).
__device__ __forceinline__ uint32_t count_before(const Plan& p, uint32_t c0, uint32_t c1, bool earlier, uint64_t a,
                                                 uint64_t A, uint32_t lo, uint32_t hi) {
    const uint64_t base = p.gpre[c0];
    const uint64_t A2 = p.gpre[c1] - base;
    while (lo < hi) {
        const uint32_t mid = (lo + hi) >> 1;
        const uint64_t a2 = p.gpre[c0 + mid] - base;
        const int c = cmp_mul128(a2, A, a, A2);
        const bool before = earlier ? (c <= 0) : (c < 0);
        if (before) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

constexpr uint32_t MERGE_K = 128;  // other strata bracketed per block at once (two threads each)

// A block whose documents all lie in one group first finds, for every other
// stratum, the counts before its first and its last document (they bound
// every count in between: the fraction grows with the position in the group);
// each thread then searches only between them.  Blocks across a group
// boundary search every stratum in full.
__global__ __launch_bounds__(256) void k_merge(Plan p, const uint32_t* val) {
    __shared__ uint32_t s_lo[MERGE_K], s_hi[MERGE_K];
    const uint64_t i0 = (uint64_t)blockIdx.x * blockDim.x;
    const uint64_t i = i0 + threadIdx.x;
    const uint64_t ilast = min((uint64_t)p.n_kept, i0 + blockDim.x) - 1;  // the block's last document
    const uint32_t gf = p.group[val[i0]], gl = p.group[val[ilast]];
    const bool one_group = gf == gl;  // uniform across the block
    const bool active = i < p.n_kept;
    const uint32_t d = active ? val[i] : val[ilast];
    const uint32_t g = p.group[d];
    const uint32_t s = p.source[d];
    // merge unit: the (stream, arrival) of the document; its strata are groups g0 .. g0+K−1
    const uint32_t u = s * p.n_seg + (p.n_seg > 1 ? p.segment[d] : 0u);
    const uint32_t g0 = p.gbase[u], K = p.n_strata[s], k = g - g0;
    const uint32_t b0 = p.group_start[g];
    const uint64_t A = p.gpre[p.group_start[g + 1]] - p.gpre[b0];
    auto frac = [&](uint64_t j) { return p.gpre[j] - p.gpre[b0]; };  // consumed tokens before element j
    const uint64_t a = frac(active ? i : ilast);
    uint64_t rank = (active ? i : ilast) - b0;
    uint64_t before = a;  // tokens of the unit's documents merged before this one: own stratum first
    for (uint32_t kb = 0; kb < K; kb += MERGE_K) {
        if (one_group) {
            __syncthreads();  // the previous chunk's bounds are read
            const uint32_t t = threadIdx.x >> 1, end = threadIdx.x & 1u;
            const uint32_t k2 = kb + t;
            if (t < MERGE_K && k2 < K && k2 != k) {
                const uint32_t c0 = p.group_start[g0 + k2], c1 = p.group_start[g0 + k2 + 1];
                const uint32_t r = c0 == c1 ? 0u
                                            : count_before(p, c0, c1, k2 < k, frac(end ? ilast : i0), A, 0u, c1 - c0);
                if (end) s_hi[t] = r;
                else s_lo[t] = r;
            }
            __syncthreads();
        }
        const uint32_t kend = min(K, kb + MERGE_K);
        for (uint32_t k2 = kb; k2 < kend; ++k2) {
            if (k2 == k) continue;
            const uint32_t c0 = p.group_start[g0 + k2], c1 = p.group_start[g0 + k2 + 1];
            if (c0 == c1) continue;
            const uint32_t lo = one_group ? s_lo[k2 - kb] : 0u, hi = one_group ? s_hi[k2 - kb] : c1 - c0;
            const uint32_t n = count_before(p, c0, c1, k2 < k, a, A, lo, hi);
            rank += n;
            before += p.gpre[c0 + n] - p.gpre[c0];
        }
    }
    if (blockIdx.x == 0)  // each stream's first position in the merged order (a stream's first arrival)
        for (uint32_t x = threadIdx.x; x <= p.S; x += blockDim.x) p.src_doc_start[x] = p.group_start[p.gbase[x * p.n_seg]];
    if (!active) return;
    const uint64_t at = p.group_start[g0] + rank;
    if (at < p.n_kept) {
        p.order[at] = d;
        // the token prefix of the merged order: the units before this one (their groups come first in
        // the sorted order, so gpre counts them), then this unit's documents merged before this one
        p.opre[at] = p.gpre[p.group_start[g0]] + before;
    } else {
        atomicOr(p.err, ERR_INTERNAL);
    }
    if (i == p.n_kept - 1) p.opre[p.n_kept] = p.gpre[p.n_kept];
}

__global__ void k_src_doc_start(Plan p) {
    const uint32_t s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s <= p.S) p.src_doc_start[s] = p.group_start[p.gbase[s * p.n_seg]];  // a stream's first arrival
    if (s == 0) p.opre[0] = 0;  // no kept document
}

// ------------------------------------------------------------------ A5 pieces
// A document of L ≤ T tokens is one piece; a longer one is ⌊L/T⌋ pieces of T
// and a tail piece (config "long-context branch": split at T).
__global__ __launch_bounds__(256) void k_pieces(Plan p) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blockIdx.x == 0)  // each stream's first piece
        for (uint32_t x = threadIdx.x; x <= p.S; x += blockDim.x) p.src_piece_start[x] = p.piece_start[p.src_doc_start[x]];
    if (i >= p.n_kept) return;
    const uint32_t d = p.order[i];
    const uint32_t q0 = p.piece_start[i];
    const uint64_t n_pieces = p.n_pieces_dev ? *p.n_pieces_dev : p.n_pieces;
    if (d >= p.n_docs || n_pieces > p.cap_pieces || p.piece_start[i + 1] > n_pieces) {
        atomicOr(p.err, ERR_INTERNAL);
        return;
    }
    const uint64_t L = p.offsets[d + 1] - p.offsets[d];
    const uint32_t np = p.piece_start[i + 1] - q0;
    const uint64_t pre = p.opre[i];
    // with a stream start: the document's tokens before it are already consumed
    uint64_t o0 = 0, cut = 0;
    const uint64_t x0 = pre - p.opre[p.src_doc_start[p.source[d]]];  // stream position of the first token
    if (p.start_tok) {
        cut = p.start_tok[p.source[d]];
        o0 = cut > x0 ? (cut - x0 < L ? cut - x0 : L) : 0;
    }
    if (!p.wrap) {
        for (uint32_t r = 0; r < np; ++r) {
            const uint64_t o = o0 + (uint64_t)r * p.T;
            const uint32_t q = q0 + r;
            p.pc_doc[q] = d;
            p.pc_off[q] = (uint32_t)o;
            p.pc_len[q] = (uint32_t)((L - o) < p.T ? (L - o) : p.T);
            p.pc_pre[q] = pre + o;
        }
    } else {
        // wrap: cut where the stream (from its start) crosses a multiple of T
        uint64_t x = x0 + o0 - cut;  // stream position of the first token to cut
        uint64_t o = o0;
        for (uint32_t r = 0; r < np; ++r) {
            const uint64_t room = p.T - x % p.T;
            const uint64_t len = (L - o) < room ? (L - o) : room;
            const uint32_t q = q0 + r;
            p.pc_doc[q] = d;
            p.pc_off[q] = (uint32_t)o;
            p.pc_len[q] = (uint32_t)len;
            p.pc_pre[q] = pre + o;
            o += len;
            x += len;
        }
        if (o != L) atomicOr(p.err, ERR_INTERNAL);  // piece count and cut disagree
    }
    if (i == p.n_kept - 1) p.pc_pre[n_pieces] = p.opre[p.n_kept];
}

__global__ void k_src_piece_start(Plan p) {
    const uint32_t s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s <= p.S) p.src_piece_start[s] = p.piece_start[p.src_doc_start[s]];
}

// ------------------------------------------------------------------ A5 next-fit
// Linnet Training, Supervised fine-tuning: windows of exactly T positions,
// padding the rest; NeuronSpark-Trainer README, Concepts: cut at document
// ends.  Next-fit in order: a window that starts at piece q holds pieces
// q … next(q)−1 with next(q) = max{ j : pre[j] − pre[q] ≤ T }.  Window starts
// of a source are next^w(first piece), w = 0, 1, …; they are found by binary
// lifting: jump[l][q] = next^(2^l)(q), END once past the source.
__global__ __launch_bounds__(256) void k_next(Plan p) {
    const uint64_t q = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= plan_pieces(p)) return;
    const uint32_t s = upper_bound_u64(p.src_piece_start, p.S + 1, q) - 1;
    const uint64_t pe = p.src_piece_start[s + 1];
    const uint64_t base = p.pc_pre[q];
    // token position where piece j starts; at the source's end, where its last piece ends (the next
    // stream's first piece can start later in the order: documents before a stream start have none)
    auto at = [&](uint64_t j) { return j < pe ? p.pc_pre[j] : p.pc_pre[pe - 1] + p.pc_len[pe - 1]; };
    uint64_t lo = q + 1, hi = q + p.T;  // a window holds at most T pieces
    if (hi > pe) hi = pe;
    // largest j in [lo, hi] with at(j) − base ≤ T  (at(q+1) − base ≤ T always)
    while (lo < hi) {
        const uint64_t mid = (lo + hi + 1) >> 1;
        if (at(mid) - base <= p.T) lo = mid;
        else hi = mid - 1;
    }
    p.jump[q] = (lo == pe) ? END : (uint32_t)lo;
}

// Levels l+1 .. l+k (k <= 3) from level l in one launch: level l+i is
// next^(2^(l+i)) = level l applied 2^i times, so a thread follows level l
// from q and records every power-of-two step (2, 4, 8 lookups).
__global__ __launch_bounds__(256) void k_lift(Plan p, const uint32_t* lev, uint32_t* out, uint64_t stride,
                                              uint32_t k) {
    const uint64_t q = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= plan_pieces(p)) return;
    uint32_t x = (uint32_t)q;
    uint32_t steps = 0;
    for (uint32_t i = 1; i <= k; ++i) {
        for (const uint32_t target = 1u << i; steps < target; ++steps) x = (x == END) ? END : lev[x];
        out[(uint64_t)(i - 1) * stride + q] = x;
    }
}

// windows per source by lifting from its first piece, then their prefix
__global__ __launch_bounds__(1024) void k_window_count(Plan p) {
    extern __shared__ uint64_t m[];  // [S]
    for (uint32_t s = threadIdx.x; s < p.S; s += blockDim.x) {
        const uint64_t a = p.src_piece_start[s], b = p.src_piece_start[s + 1];
        uint64_t M = 0;
        if (a < b) {
            uint32_t cur = (uint32_t)a;
            M = 1;
            for (int l = (int)p.levels - 1; l >= 0; --l) {
                const uint32_t nx = p.jump[(uint64_t)l * p.cap_pieces + cur];
                if (nx != END) {
                    cur = nx;
                    M += 1ull << l;
                }
            }
        }
        m[s] = M;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t run = 0;
        for (uint32_t s = 0; s < p.S; ++s) {
            p.src_win_start[s] = run;
            run += m[s];
        }
        p.src_win_start[p.S] = run;
    }
}

__global__ __launch_bounds__(256) void k_windows(Plan p) {
    const uint64_t gw = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t n_windows = plan_windows(p);
    if (gw >= n_windows) return;
    const uint32_t s = upper_bound_u64(p.src_win_start, p.S + 1, gw) - 1;
    const uint64_t w = gw - p.src_win_start[s];
    uint32_t cur = (uint32_t)p.src_piece_start[s];
    for (uint32_t l = 0; l < p.levels; ++l)
        if ((w >> l) & 1) cur = p.jump[(uint64_t)l * p.cap_pieces + cur];
    p.win_first[gw] = cur;
    if (gw == n_windows - 1) p.win_first[n_windows] = (uint32_t)plan_pieces(p);
}

// Wrap packing: source s has ceil(Λ_s / T) windows (Λ_s its kept tokens), and
// window w of s starts at the piece whose stream position is w·T.
__global__ __launch_bounds__(1024) void k_wrap_window_count(Plan p) {
    if (threadIdx.x != 0) return;
    uint64_t run = 0;
    for (uint32_t s = 0; s < p.S; ++s) {
        p.src_win_start[s] = run;
        uint64_t lam = p.opre[p.src_doc_start[s + 1]] - p.opre[p.src_doc_start[s]];
        if (p.start_tok) lam = p.start_tok[s] < lam ? lam - p.start_tok[s] : 0;  // tokens from the stream's start
        run += (lam + p.T - 1) / p.T;
    }
    p.src_win_start[p.S] = run;
}

__global__ __launch_bounds__(256) void k_wrap_windows(Plan p) {
    const uint64_t q = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t n_pieces = plan_pieces(p), n_windows = plan_windows(p);
    if (q >= n_pieces) return;
    const uint32_t s = upper_bound_u64(p.src_piece_start, p.S + 1, q) - 1;
    // stream position of the piece, from the stream's start
    const uint64_t y = p.pc_pre[q] - p.opre[p.src_doc_start[s]] - (p.start_tok ? p.start_tok[s] : 0);
    if (y % p.T == 0) {
        const uint64_t gw = p.src_win_start[s] + y / p.T;
        if (gw < n_windows) p.win_first[gw] = (uint32_t)q;
        else atomicOr(p.err, ERR_INTERNAL);
    }
    if (q == n_pieces - 1) p.win_first[n_windows] = (uint32_t)n_pieces;
}

// offsets of pieces in their window; real and learned positions per window
// (Linnet Training: a prompted example learns only its completion).  Also the
// emission view of each piece: window position t of the piece holds token
// base + t (base = off[d] + o − f, modulo 2^64) and learns iff t ≥ mfrom
// (mfrom = f + min(max(prompt_len − o, 0), len), so t < f + len never learns
// when the prompt covers the piece).
__global__ __launch_bounds__(256) void k_window_stats(Plan p) {
    const uint64_t gw = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gw >= plan_windows(p)) return;
    const uint32_t q0 = p.win_first[gw], q1 = p.win_first[gw + 1];
    if (q0 >= q1 || q1 > plan_pieces(p)) {
        atomicOr(p.err, ERR_INTERNAL);
        p.win_real[gw] = 0;
        p.win_learn[gw] = 0;
        return;
    }
    uint32_t f = 0, learn = 0;
    for (uint32_t q = q0; q < q1; q += 4) {  // four pieces at a time, every load before any store
        uint32_t o[4], len[4], d[4], pl[4];
        uint64_t od[4];
#pragma unroll
        for (uint32_t u = 0; u < 4; ++u) {
            const bool in = q + u < q1;
            o[u] = in ? p.pc_off[q + u] : 0u;
            len[u] = in ? p.pc_len[q + u] : 0u;
            d[u] = in ? p.pc_doc[q + u] : 0u;
        }
#pragma unroll
        for (uint32_t u = 0; u < 4; ++u) {
            const bool in = q + u < q1;
            pl[u] = in && p.prompt_len ? p.prompt_len[d[u]] : 0u;
            od[u] = in ? p.offsets[d[u]] : 0ull;
        }
#pragma unroll
        for (uint32_t u = 0; u < 4; ++u) {
            if (q + u >= q1) break;
            p.pc_woff[q + u] = f;
            const uint64_t from = o[u] > pl[u] ? o[u] : pl[u];
            if ((uint64_t)o[u] + len[u] > from) learn += (uint32_t)((uint64_t)o[u] + len[u] - from);
            const uint64_t base = od[u] + o[u] - f;
            const uint32_t lead = (uint32_t)(from - o[u] < len[u] ? from - o[u] : len[u]);  // prompt positions
            p.pc_emit[q + u] = make_uint4((uint32_t)base, (uint32_t)(base >> 32), d[u], f + lead);
            f += len[u];
        }
    }
    p.win_real[gw] = f;
    p.win_learn[gw] = learn;
}

// ------------------------------------------------------------------ A6 mixture
// NeuronSpark-Trainer README, Concepts: every update holds each source within
// two samples of its recipe share.  Largest remainder: n_s = ⌊B·w_s/W⌋, the
// leftover seats one each to the largest remainders B·w_s mod W, ties to the
// lower source; the same n_s for every update (within one of the quota).

// floor and remainder of (hi:lo) / W for hi < W (so the quotient fits 64 bits)
__device__ inline uint64_t div128(uint64_t hi, uint64_t lo, uint64_t W, uint64_t* rem) {
    uint64_t q = 0, r = hi;
    for (int b = 63; b >= 0; --b) {
        const bool carry = (r >> 63) != 0;
        r = (r << 1) | ((lo >> b) & 1ull);
        q <<= 1;
        if (carry || r >= W) {
            r -= W;
            q |= 1ull;
        }
    }
    *rem = r;
    return q;
}

__global__ __launch_bounds__(1024) void k_apportion(Plan p, uint64_t W, uint32_t B, uint32_t* n_out,
                                                    uint32_t* nstart) {
    extern __shared__ uint64_t sh[];  // rem[S] then n[S] (32-bit)
    uint64_t* rem = sh;
    uint32_t* nn = reinterpret_cast<uint32_t*>(sh + p.S);
    __shared__ uint64_t given_s;
    if (threadIdx.x == 0) given_s = 0;
    __syncthreads();
    for (uint32_t s = threadIdx.x; s < p.S; s += blockDim.x) {
        const uint64_t w = p.weight[s];
        const uint64_t hi = __umul64hi((uint64_t)B, w), lo = (uint64_t)B * w;
        uint64_t r;
        const uint64_t n = div128(hi, lo, W, &r);  // hi < W since B·w < B·W
        rem[s] = r;
        nn[s] = (uint32_t)n;
        atomicAdd((unsigned long long*)&given_s, (unsigned long long)n);
    }
    __syncthreads();
    const uint64_t left = (uint64_t)B - given_s;
    for (uint32_t s = threadIdx.x; s < p.S; s += blockDim.x) {
        uint64_t rank = 0;
        for (uint32_t t = 0; t < p.S; ++t)
            rank += (rem[t] > rem[s] || (rem[t] == rem[s] && t < s)) ? 1 : 0;
        n_out[s] = (uint32_t)(nn[s] + (rank < left ? 1 : 0));
    }
    __syncthreads();
    if (threadIdx.x == 0 && nstart) {
        uint32_t run = 0;
        for (uint32_t s = 0; s < p.S; ++s) {
            nstart[s] = run;
            run += n_out[s];
        }
        nstart[p.S] = run;
    }
}

// Slot order inside an update: items (s, k), k < n_s, by (2k+1)/(2n_s), ties
// to the lower source (Sainte-Laguë order), so the sources are spread over
// the update.  Position of (s, k) = number of items ordered before it,
// counted in closed form per source.  Item u of the update (sources in
// order, nstart = exclusive prefix of the counts) → (s, k, position).
__device__ inline uint64_t slot_item(const uint32_t* n, const uint32_t* nstart, uint32_t S, uint32_t u,
                                     uint32_t* s_out, uint32_t* k_out) {
    uint32_t lo = 0, hi = S;  // source s with nstart[s] ≤ u < nstart[s+1]
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (nstart[mid] <= u) lo = mid;
        else hi = mid;
    }
    uint32_t s = lo;
    while (nstart[s + 1] <= u) ++s;  // skip sources with n = 0
    const uint32_t k = u - nstart[s];
    const uint64_t ns = n[s];
    uint64_t pos = k;
    for (uint32_t s2 = 0; s2 < S; ++s2) {
        const uint64_t n2 = n[s2];
        if (s2 == s || n2 == 0) continue;
        const uint64_t X = (2ull * k + 1) * n2;   // compare (2k'+1)·n_s against X
        const uint64_t F = (s2 < s) ? X / ns : (X - 1) / ns;  // largest admissible odd bound
        uint64_t c = (F + 1) / 2;
        if (c > n2) c = n2;
        pos += c;
    }
    *s_out = s;
    *k_out = k;
    return pos;
}

__global__ __launch_bounds__(256) void k_slots(Plan p, const uint32_t* nstart) {
    const uint32_t u = blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= p.B) return;
    uint32_t s, k;
    const uint64_t pos = slot_item(p.n_upd, nstart, p.S, u, &s, &k);
    if (pos < p.B) {
        p.slot_src[pos] = s;
        p.slot_k[pos] = k;
    } else {
        atomicOr(p.err, ERR_INTERNAL);
    }
}

// ------------------------------------------------------------------ cumulative mixture
// One workgroup, thread s = source s (S ≤ CUM_MAX_S), one update after the
// other.  After update u, source s has taken A_s with floor(q) ≤ A_s ≤ ceil(q),
// q = (u+1)·B·w_s/W, kept as q = fl + rm/W with B·w_s = qB·W + rB added per
// update.  The windows due by update u are those up to fl (fl − A_s of them,
// all taken); the only other released window of s is window fl+1 when
// rm ≠ 0 and A_s ≤ fl, due by update δ = ceil((fl+1)·W/(B·w_s)) − 1, which
// depends on fl alone: u + 1 when B·w_s ≥ W, else u + ceil((W − rm)/(B·w_s))
// evaluated when fl last changed.  The B − Σ(fl − A_s)⁺ remaining seats R go
// to the candidates with the smallest (δ, s) (earliest deadline first): every
// wave finds the threshold key κ, the smallest with at least R candidates at
// or below it, by galloping and bisecting over the due update with ballot
// counts of the ROWS key rows (a row = the keys of 64 consecutive sources),
// and a candidate takes a seat when its key is below κ or equals κ within
// the first R − #(keys < κ) of those ties by source.  The schedule stops
// before the first update after which a source would exceed the windows it
// has left, or after cap updates.
// ROWS = 1 (S ≤ 64): one wavefront, no LDS and no barrier.  ROWS > 1: each
// update publishes the keys and the waves' sums in LDS behind one barrier
// (double-buffered by the update's parity, so no second barrier guards their
// reuse); whether an update fits the windows left is read at the next
// update's barrier, and an update that does not fit is undone (its table row
// lies past the cycle's U).
constexpr uint32_t CUM_MAX_S = 1024;

template <uint32_t ROWS>
__global__ __launch_bounds__(ROWS * WAVE) void k_cumulative(Plan p, uint64_t W, uint64_t cap) {
    constexpr bool ONE = ROWS == 1;
    __shared__ uint64_t key[ONE ? 1 : 2][ONE ? 1 : ROWS * WAVE];
    __shared__ uint64_t part[ONE ? 1 : 2][3][ONE ? 1 : ROWS];
    const uint32_t s = threadIdx.x, lane = s & (WAVE - 1), wv = s / WAVE;
    const bool on = s < p.S;
    const uint64_t w = on ? p.weight[s] : 0;
    // the update's step of the quota, B_u·w_s = qB·W + rB (recomputed when the batch changes)
    uint64_t bw_hi = 0, bw = 0, rB = 0, qB = 0;
    bool step_ge_W = false;  // fl grows every update
    uint32_t Bu = 0;
    const uint64_t rem = on ? p.cum_rem[s] : ~0ull;
    uint64_t fl = 0, rm = 0, A = 0, U = 0, due = 0;
    uint64_t A_prev = 0;  // ROWS > 1: A before the update whose fit is not yet known
    bool bad = false, over_prev = false, undone = false;
    if (on) p.cum_A[s] = 0;
    uint64_t u = 0;
    for (; u < cap; ++u) {
        const uint32_t Bn = (p.ramp ? p.upd_B[u] : p.B) / p.lanes;  // this lane's seats in update u
        if (Bn != Bu) {  // uniform: the same batch for every source
            Bu = Bn;
            bw_hi = __umul64hi((uint64_t)Bu, w);
            bw = (uint64_t)Bu * w;
            rB = 0;
            qB = w ? div128(bw_hi, bw, W, &rB) : 0;  // bw_hi < W since B·w < 2^20·W
            step_ge_W = bw_hi != 0 || bw >= W;
        }
        bool moved = false;
        if (w) {  // q ← q + B·w_s/W
            uint64_t r2 = rm + rB;
            const bool carry = r2 < rm;
            fl += qB;
            moved = qB != 0;
            if (carry || r2 >= W) {
                r2 -= W;
                fl += 1;
                moved = true;
            }
            rm = r2;
        }
        const uint64_t m = fl > A ? fl - A : 0;
        const bool cand = w != 0 && rm != 0 && A <= fl;
        if (w && (moved || u == 0)) {  // the formula holds for rm = 0 too: δ of window fl+1
            if (!p.ramp) {
                if (step_ge_W) {
                    due = u + 1;
                } else {
                    const uint64_t gap = W - rm;
                    due = u + gap / bw + (gap % bw ? 1 : 0);
                }
            } else {
                // the first v > u with H(v+1)·w_s ≥ (fl+1)·W, H(v) = seats before update v from the
                // ramp's spans (the last without end, so the due does not depend on the cycle's length)
                const unsigned __int128 goal = (unsigned __int128)(fl + 1) * W;
                auto reached = [&](uint64_t v) {
                    uint32_t lo = 0, hi = p.n_spans;  // span of update v
                    while (hi - lo > 1) {
                        const uint32_t mid = (lo + hi) >> 1;
                        if (p.spans[mid].first <= v) lo = mid;
                        else hi = mid;
                    }
                    const RampSpan& r = p.spans[lo];
                    const uint64_t seats = (r.slot0 + (v + 1 - r.first) * r.B) / p.lanes;  // this lane's H(v+1)
                    return (unsigned __int128)seats * w >= goal;
                };
                uint64_t lo = u, hi = u + 1, step = 1;  // not reached(u): fl is the quota's floor after u
                while (!reached(hi)) {                  // gallop (dues lie within 2^62 updates: shares ≥ 2^-62)
                    lo = hi;
                    step *= 2;
                    hi = lo + step;
                }
                while (hi - lo > 1) {  // reached(hi), not reached(lo)
                    const uint64_t mid = lo + (hi - lo) / 2;
                    if (reached(mid)) hi = mid;
                    else lo = mid;
                }
                due = hi;
            }
        }
        const uint64_t k = cand ? due : ~0ull;
        uint64_t sm = wave_sum_u64(m), nc = (uint64_t)__popcll(__ballot(cand));
        const uint32_t par = (uint32_t)(u & 1);
        if (!ONE) {
            key[par][s] = k;
            if (lane == 0) {
                part[par][0][wv] = sm;
                part[par][1][wv] = nc;
                part[par][2][wv] = over_prev ? 1 : 0;  // the previous update took more than a source has
            }
            __syncthreads();
            sm = 0;
            nc = 0;
            uint64_t ovp = 0;
#pragma unroll
            for (uint32_t i = 0; i < ROWS; ++i) {
                sm += part[par][0][i];
                nc += part[par][1][i];
                ovp += part[par][2][i];
            }
            if (ovp) {  // update u − 1 does not fit: the cycle ends after u − 1 updates
                A = A_prev;
                undone = true;
                break;
            }
            U = u;
        }
        if (sm > Bu || nc < Bu - sm) {  // the schedule's guarantee failed
            bad = true;
            break;
        }
        const uint64_t R = Bu - sm;
        bool take = false;
        if (R) {
            uint64_t kr[ROWS];  // every wave holds all key rows (non-candidates ~0) and finds the same κ
#pragma unroll
            for (uint32_t r = 0; r < ROWS; ++r) kr[r] = ONE ? k : key[par][r * WAVE + lane];
            auto count_le = [&](uint64_t thr) {
                uint64_t c = 0;
#pragma unroll
                for (uint32_t r = 0; r < ROWS; ++r) c += (uint64_t)__popcll(__ballot(kr[r] <= thr));
                return c;
            };
            // A candidate's window fl+1 is due after update u (fl would have moved in its due
            // update), so no key is at most u: count_le(u) = 0 < R.  Keys stay below 2^64 − 1
            // (dues lie within 2^62 updates), where the count is nc ≥ R.
            constexpr uint64_t TOP = ~0ull - 1;
            uint64_t lo = u, hi = u, below = 0, step = 1;
            for (;;) {  // gallop: count_le(lo) = below < R
                hi = step > TOP - lo ? TOP : lo + step;
                const uint64_t c = count_le(hi);
                if (c >= R) break;
                lo = hi;
                below = c;
                step <<= 1;
            }
            while (hi - lo > 1) {  // count_le(lo) = below < R ≤ count_le(hi)
                const uint64_t mid = lo + (hi - lo) / 2;
                const uint64_t c = count_le(mid);
                if (c >= R) {
                    hi = mid;
                } else {
                    lo = mid;
                    below = c;
                }
            }
            // κ = hi; the ties at κ take the R − below seats left, lower sources first
            const bool tie = cand && k == hi;
            uint64_t rank = (uint64_t)__popcll(__ballot(tie) & ((1ull << lane) - 1ull));
#pragma unroll
            for (uint32_t r = 0; r + 1 < ROWS; ++r) rank += r < wv ? (uint64_t)__popcll(__ballot(kr[r] == hi)) : 0;
            take = cand && (k < hi || (tie && rank < R - below));
        }
        const uint64_t An = A + m + (take ? 1 : 0);
        if (ONE) {
            if (__ballot(An > rem)) break;
            A = An;
            U = u + 1;
        } else {  // the fit is read at the next update's barrier (or after the loop)
            over_prev = __ballot(An > rem) != 0;
            A_prev = A;
            A = An;
        }
        if (on) p.cum_A[(u + 1) * p.S + s] = (uint32_t)An;
    }
    if (!ONE && !bad && !undone && u == cap && cap) {  // the last update's fit
        const uint32_t par = (uint32_t)(cap & 1);
        if (lane == 0) part[par][2][wv] = over_prev ? 1 : 0;
        __syncthreads();
        uint64_t ovp = 0;
#pragma unroll
        for (uint32_t i = 0; i < ROWS; ++i) ovp += part[par][2][i];
        if (ovp) A = A_prev;
        else U = cap;
    }
    if (on) p.cum_out[s] = A;
    if (s == 0) p.cum_out[p.S] = U;
    if (bad && s == 0) atomicOr(p.err, ERR_INTERNAL);
}

// Integral quotas: when every update's seats times every weight is a multiple
// of W (one source, or shares that divide the batch), every quota is an
// integer, no window is ever taken ahead of its quota, and the schedule above
// is A_s(u) = H(u)·w_s/W exactly, H(u) being the lane's seats before update u.
// Then no update-by-update loop is needed: one thread per source finds the
// last update its windows cover (A_s is nondecreasing in u), the minimum over
// sources (at most cap) is the cycle's U, and a grid writes the table.
__device__ inline uint64_t lane_seats_before(const Plan& p, uint64_t u) {
    if (!p.ramp) return u * (uint64_t)(p.B / p.lanes);
    uint32_t lo = 0, hi = p.n_spans;  // span of update u
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (p.spans[mid].first <= u) lo = mid;
        else hi = mid;
    }
    const RampSpan& r = p.spans[lo];
    return (r.slot0 + (u - r.first) * r.B) / p.lanes;
}

__device__ inline uint64_t integral_quota(const Plan& p, uint64_t u, uint64_t w, uint64_t W) {
    const uint64_t H = lane_seats_before(p, u);
    uint64_t r;
    return w ? div128(__umul64hi(H, w), H * w, W, &r) : 0;  // the quotient is at most H: hi < W
}

__global__ __launch_bounds__(1024) void k_cum_integral_U(Plan p, uint64_t W, uint64_t cap) {
    __shared__ unsigned long long U;
    if (threadIdx.x == 0) U = cap;
    __syncthreads();
    for (uint32_t s = threadIdx.x; s < p.S; s += blockDim.x) {
        const uint64_t w = p.weight[s], rem = p.cum_rem[s];
        if (w == 0 || integral_quota(p, cap, w, W) <= rem) continue;
        uint64_t lo = 0, hi = cap;  // A_s(lo) ≤ rem < A_s(hi)
        while (hi - lo > 1) {
            const uint64_t mid = lo + (hi - lo) / 2;
            if (integral_quota(p, mid, w, W) <= rem) lo = mid;
            else hi = mid;
        }
        atomicMin(&U, (unsigned long long)lo);
    }
    __syncthreads();
    for (uint32_t s = threadIdx.x; s < p.S; s += blockDim.x) p.cum_out[s] = integral_quota(p, U, p.weight[s], W);
    if (threadIdx.x == 0) p.cum_out[p.S] = U;
}

__global__ __launch_bounds__(256) void k_cum_integral_A(Plan p, uint64_t W, uint64_t cap) {
    const uint64_t x = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= (cap + 1) * p.S) return;
    const uint64_t u = x / p.S;
    const uint32_t s = (uint32_t)(x - u * p.S);
    if (u > p.cum_out[p.S]) return;
    p.cum_A[x] = (uint32_t)integral_quota(p, u, p.weight[s], W);
}

// Slot table of every update of the cycle: block u, counts
// A(u+1) − A(u) in Sainte-Laguë order; cslot_i = A_s(u) + k.
__global__ __launch_bounds__(256) void k_cum_slots(Plan p) {
    extern __shared__ uint32_t csh[];  // n[S], nstart[S+1], base[S] over the real sources
    const uint32_t S = p.S_real, L = p.lanes;  // block (u, l): lane l's slots of update u
    uint32_t* n = csh;
    uint32_t* ns = csh + S;
    uint32_t* base = csh + 2 * S + 1;
    const uint64_t u = blockIdx.x;
    const uint32_t l = blockIdx.y;
    const uint32_t Bu = (p.ramp ? p.upd_B[u] : p.B) / L;
    const uint64_t x0 = (p.ramp ? p.upd_slot0[u] : u * p.B) + (uint64_t)l * Bu;  // the lane's first slot
    for (uint32_t s = threadIdx.x; s < S; s += blockDim.x) {
        const uint32_t v = s * L + l;  // stream (source s, lane l)
        const uint32_t a0 = p.cum_A[u * p.S + v], a1 = p.cum_A[(u + 1) * p.S + v];
        n[s] = a1 - a0;
        base[s] = a0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t run = 0;
        for (uint32_t s = 0; s < S; ++s) {
            ns[s] = run;
            run += n[s];
        }
        ns[S] = run;
        if (run != Bu) atomicOr(p.err, ERR_INTERNAL);
    }
    __syncthreads();
    if (ns[S] != Bu) return;
    for (uint32_t t = threadIdx.x; t < Bu; t += blockDim.x) {
        uint32_t s, k;
        const uint64_t pos = slot_item(n, ns, S, t, &s, &k);
        if (pos < Bu) {
            p.cslot_src[x0 + pos] = s * L + l;
            p.cslot_i[x0 + pos] = base[s] + k;
        } else {
            atomicOr(p.err, ERR_INTERNAL);
        }
    }
}

// ------------------------------------------------------------------ checks
// two 64-bit sums for the plan digest; integer sums are order-free, so a
// grid-stride loop with one atomic per block gives the exact value
__device__ inline void block_add2(uint64_t x, uint64_t y, uint64_t* dst) {
    __shared__ uint64_t part[2][256 / WAVE];
    x = wave_sum_u64(x);
    y = wave_sum_u64(y);
    if ((threadIdx.x & 63) == 0) {
        part[0][threadIdx.x / WAVE] = x;
        part[1][threadIdx.x / WAVE] = y;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t a = 0, b = 0;
        for (int w = 0; w < 256 / WAVE; ++w) {
            a += part[0][w];
            b += part[1][w];
        }
        if (a) atomicAdd((unsigned long long*)&dst[0], (unsigned long long)a);
        if (b) atomicAdd((unsigned long long*)&dst[1], (unsigned long long)b);
    }
}

__global__ __launch_bounds__(256) void k_checks(Plan p) {
    uint64_t oc = 0, hc = 0;
    const uint64_t n = p.n_docs > p.n_kept ? p.n_docs : p.n_kept;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x) {
        if (i < p.n_kept) oc += mix64((i << 32) ^ (uint64_t)p.order[i]);
        if (i < p.n_docs && p.keep[i]) hc += p.hash[i];
    }
    block_add2(oc, hc, p.checks);
}

// The cycle's sums over its slots (cyc_sums zeroed before); block 0 also
// writes each stream's token, in its merged order, where window next_win[s]
// begins (pc_pre holds the order's token prefix), or the stream's total when
// next_win[s] = ~0 (used up): where the next cycle starts.
__global__ __launch_bounds__(256) void k_cycle_sums(Plan p, uint64_t total, const uint64_t* next_win,
                                                    uint64_t* stream_next) {
    // test option: report an internal failure of the cycle (pack_cycle must fail)
    if ((p.test_opts & TEST_CYCLE_FAULT) && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(p.err, ERR_INTERNAL);
    if (blockIdx.x == 0)
        for (uint32_t s = threadIdx.x; s < p.S; s += blockDim.x) {
            const uint64_t base = p.opre[p.src_doc_start[s]];
            const uint64_t w = next_win[s];
            stream_next[s] = w == ~0ull ? p.opre[p.src_doc_start[s + 1]] - base : p.pc_pre[p.win_first[w]] - base;
        }
    uint64_t real = 0, learn = 0;
    for (uint64_t idx = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t gw = p.tabled ? window_of_slot(p, idx) : window_of(p, idx / p.B, (uint32_t)(idx % p.B));
        real += p.win_real[gw];
        learn += p.win_learn[gw];
    }
    block_add2(real, learn, p.cyc_sums);
}

// ------------------------------------------------------------------ batch-size ramp
// Update u of the cycle lies in the last span whose first update is ≤ u; its
// batch, first slot and first output window follow in closed form.
__device__ inline uint32_t span_of(const RampSpan* sp, uint32_t n, uint64_t u) {
    uint32_t lo = 0, hi = n;  // sp[lo].first ≤ u < sp[hi].first
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (sp[mid].first <= u) lo = mid;
        else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(256) void k_ramp_fill(Plan p, const RampSpan* sp, uint32_t n_spans, uint64_t n_upd) {
    const uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u > n_upd) return;
    const RampSpan r = sp[span_of(sp, n_spans, u)];
    const uint64_t d = u - r.first;
    if (u < n_upd) p.upd_B[u] = r.B;
    p.upd_slot0[u] = r.slot0 + d * r.B;
    p.upd_out0[u] = r.out0 + d * (r.B / p.world);
}

// cum_A[u][s] = Σ over spans of the updates before u in the span · the span piece's n_s
__global__ __launch_bounds__(256) void k_ramp_fixed_A(Plan p, const RampSpan* sp, uint32_t n_spans,
                                                      const uint32_t* ramp_n, uint64_t U) {
    const uint64_t x = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= (U + 1) * p.S) return;
    const uint64_t u = x / p.S;
    const uint32_t s = (uint32_t)(x % p.S);
    uint64_t a = 0;
    for (uint32_t k = 0; k < n_spans && sp[k].first < u; ++k) {
        const uint64_t end = k + 1 < n_spans ? sp[k + 1].first : ~0ull;
        const uint64_t upto = u < end ? u : end;
        a += (upto - sp[k].first) * ramp_n[(uint64_t)sp[k].k * p.S + s];
    }
    p.cum_A[x] = (uint32_t)a;
}

// ------------------------------------------------------------------ lanes
// stream of each document: (source, lane d mod L) = source·L + d mod L; an id
// outside the sources stays invalid (0xFFFF) for the validation kernel
__global__ __launch_bounds__(256) void k_lane_source(const uint16_t* source, uint64_t n, uint32_t S_real,
                                                     uint32_t L, uint16_t* out) {
    const uint64_t d = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (d >= n) return;
    const uint32_t s = source[d];
    out[d] = s < S_real ? (uint16_t)(s * L + (uint32_t)(d % L)) : (uint16_t)0xFFFF;
}

// every lane the same counts (n_upd of stream s·L + l = n_real[s]) and slot
// table (lane l's slots l·B/L .. hold the one-lane table's sources in lane l)
__global__ __launch_bounds__(256) void k_lane_expand(Plan p, const uint32_t* n_real, const uint32_t* lane_src,
                                                     const uint32_t* lane_k) {
    const uint32_t x = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t L = p.lanes, BL = p.B / L;
    if (x < p.S) p.n_upd[x] = n_real[x / L];
    if (x < p.B) {
        p.slot_src[x] = lane_src[x % BL] * L + x / BL;
        p.slot_k[x] = lane_k[x % BL];
    }
}

// every lane follows the one-lane schedule: cum_A[u][s·L + l] = cum_Ar[u][s]
__global__ __launch_bounds__(256) void k_cum_expand(Plan p, const uint32_t* cum_Ar, uint64_t U) {
    const uint64_t x = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= (U + 1) * p.S) return;
    const uint64_t u = x / p.S;
    const uint32_t v = (uint32_t)(x % p.S);
    p.cum_A[x] = cum_Ar[u * p.S_real + v / p.lanes];
}

inline uint32_t blocks_for(uint64_t n, uint32_t b = 256) { return (uint32_t)((n + b - 1) / b); }

}  // namespace

void launch_merge(Plan& p, hipStream_t st) {
    const uint32_t* val = p.val[p.sort_buf];
    if (p.n_kept) {
        hipLaunchKernelGGL(k_group_bounds, dim3(blocks_for(p.n_kept)), dim3(256), 0, st, val, p.group, p.n_kept, p.G,
                           p.group_start, p.order);
    } else {  // no document: every group starts (and ends) at 0
        hipLaunchKernelGGL(k_fill_u32, dim3(blocks_for(p.G + 1)), dim3(256), 0, st, p.group_start,
                           (uint64_t)p.G + 1, 0u);
    }
    scan_len_u64(val, p.offsets, p.n_kept, p.gpre, p.scan, st);
    if (p.n_kept) hipLaunchKernelGGL(k_merge, dim3(blocks_for(p.n_kept)), dim3(256), 0, st, p, val);
    else hipLaunchKernelGGL(k_src_doc_start, dim3(blocks_for(p.S + 1)), dim3(256), 0, st, p);
    DP_HIP(hipGetLastError());
}

// p.opre, the token prefix of the merged order, was written by the merge
void launch_piece_count(Plan& p, hipStream_t st) {
    if (p.wrap)
        scan_wrap_pieces_u32(p.order, p.offsets, p.opre, p.src_doc_start, p.source, p.start_tok, p.T, p.n_kept,
                             p.piece_start, p.scan, st);
    else
        scan_pieces_u32(p.order, p.offsets, p.opre, p.src_doc_start, p.source, p.start_tok, p.T, p.n_kept,
                        p.piece_start, p.scan, st);
}

void launch_pieces(Plan& p, hipStream_t st) {
    if (p.n_kept) hipLaunchKernelGGL(k_pieces, dim3(blocks_for(p.n_kept)), dim3(256), 0, st, p);
    else hipLaunchKernelGGL(k_src_piece_start, dim3(blocks_for(p.S + 1)), dim3(256), 0, st, p);
    DP_HIP(hipGetLastError());
}

// p.n_pieces: the piece count or its bound (the kernels read the count itself)
void launch_lifting(Plan& p, hipStream_t st) {
    if (p.n_pieces == 0 || p.wrap) return;  // wrap packing cuts by position, no next-fit
    hipLaunchKernelGGL(k_next, dim3(blocks_for(p.n_pieces)), dim3(256), 0, st, p);
    for (uint32_t l = 1; l < p.levels;) {  // levels l .. l+k-1 from level l-1
        const uint32_t k = p.levels - l < 3 ? p.levels - l : 3;
        hipLaunchKernelGGL(k_lift, dim3(blocks_for(p.n_pieces)), dim3(256), 0, st, p,
                           (const uint32_t*)(p.jump + (uint64_t)(l - 1) * p.cap_pieces),
                           p.jump + (uint64_t)l * p.cap_pieces, p.cap_pieces, k);
        l += k;
    }
    DP_HIP(hipGetLastError());
}

void launch_window_count(Plan& p, hipStream_t st) {
    if (p.wrap) hipLaunchKernelGGL(k_wrap_window_count, dim3(1), dim3(64), 0, st, p);
    else hipLaunchKernelGGL(k_window_count, dim3(1), dim3(1024), (size_t)p.S * sizeof(uint64_t), st, p);
    DP_HIP(hipGetLastError());
}

// p.n_pieces, p.n_windows: the counts or their bound (the kernels read the counts)
void launch_windows(Plan& p, hipStream_t st) {
    if (p.n_windows == 0) return;
    if (p.wrap) hipLaunchKernelGGL(k_wrap_windows, dim3(blocks_for(p.n_pieces)), dim3(256), 0, st, p);
    else hipLaunchKernelGGL(k_windows, dim3(blocks_for(p.n_windows)), dim3(256), 0, st, p);
    hipLaunchKernelGGL(k_window_stats, dim3(blocks_for(p.n_windows)), dim3(256), 0, st, p);
    DP_HIP(hipGetLastError());
}

void launch_mixture_w(Plan& p, uint64_t W, uint32_t* nstart, hipStream_t st) {
    hipLaunchKernelGGL(k_apportion, dim3(1), dim3(1024), (size_t)p.S * 12, st, p, W, p.B, p.n_upd, nstart);
    hipLaunchKernelGGL(k_slots, dim3(blocks_for(p.B)), dim3(256), 0, st, p, (const uint32_t*)nstart);
    DP_HIP(hipGetLastError());
}

void launch_cumulative(Plan& p, uint64_t W, uint64_t cap, bool integral, hipStream_t st) {
    if (integral) {
        hipLaunchKernelGGL(k_cum_integral_U, dim3(1), dim3(1024), 0, st, p, W, cap);
        hipLaunchKernelGGL(k_cum_integral_A, dim3(blocks_for((cap + 1) * p.S)), dim3(256), 0, st, p, W, cap);
    } else {  // rows of 64 sources, a power of two
        if (p.S > CUM_MAX_S) throw HipError{hipErrorInvalidValue, "internal: cumulative schedule over more than 1024 sources"};
        const uint32_t rows = (p.S + WAVE - 1) / WAVE;
        if (rows <= 1) hipLaunchKernelGGL(k_cumulative<1>, dim3(1), dim3(WAVE), 0, st, p, W, cap);
        else if (rows <= 2) hipLaunchKernelGGL(k_cumulative<2>, dim3(1), dim3(2 * WAVE), 0, st, p, W, cap);
        else if (rows <= 4) hipLaunchKernelGGL(k_cumulative<4>, dim3(1), dim3(4 * WAVE), 0, st, p, W, cap);
        else if (rows <= 8) hipLaunchKernelGGL(k_cumulative<8>, dim3(1), dim3(8 * WAVE), 0, st, p, W, cap);
        else hipLaunchKernelGGL(k_cumulative<16>, dim3(1), dim3(16 * WAVE), 0, st, p, W, cap);
    }
    DP_HIP(hipGetLastError());
}

void launch_cum_slots(Plan& p, uint32_t U, hipStream_t st) {
    if (U) hipLaunchKernelGGL(k_cum_slots, dim3(U, p.lanes), dim3(256), (size_t)(3 * p.S_real + 1) * 4, st, p);
    DP_HIP(hipGetLastError());
}

void launch_lane_source(const uint16_t* source, uint64_t n_docs, uint32_t S_real, uint32_t L, uint16_t* out,
                        hipStream_t st) {
    if (n_docs) hipLaunchKernelGGL(k_lane_source, dim3(blocks_for(n_docs)), dim3(256), 0, st, source, n_docs, S_real, L, out);
    DP_HIP(hipGetLastError());
}

void launch_lane_expand(Plan& p, const uint32_t* n_real, const uint32_t* lane_src, const uint32_t* lane_k,
                        hipStream_t st) {
    hipLaunchKernelGGL(k_lane_expand, dim3(blocks_for(std::max<uint64_t>(p.B, p.S))), dim3(256), 0, st, p, n_real,
                       lane_src, lane_k);
    DP_HIP(hipGetLastError());
}

void launch_cum_expand(Plan& p, const uint32_t* cum_Ar, uint64_t U, hipStream_t st) {
    hipLaunchKernelGGL(k_cum_expand, dim3(blocks_for((U + 1) * p.S)), dim3(256), 0, st, p, cum_Ar, U);
    DP_HIP(hipGetLastError());
}

void launch_apportion(Plan& p, uint64_t W, uint32_t B, uint32_t* n_out, hipStream_t st) {
    hipLaunchKernelGGL(k_apportion, dim3(1), dim3(1024), (size_t)p.S * 12, st, p, W, B, n_out, (uint32_t*)nullptr);
    DP_HIP(hipGetLastError());
}

void launch_ramp_fill(Plan& p, const RampSpan* spans, uint32_t n_spans, uint64_t n_upd, hipStream_t st) {
    hipLaunchKernelGGL(k_ramp_fill, dim3(blocks_for(n_upd + 1)), dim3(256), 0, st, p, spans, n_spans, n_upd);
    DP_HIP(hipGetLastError());
}

void launch_ramp_fixed_A(Plan& p, const RampSpan* spans, uint32_t n_spans, const uint32_t* ramp_n, uint64_t U,
                         hipStream_t st) {
    hipLaunchKernelGGL(k_ramp_fixed_A, dim3(blocks_for((U + 1) * p.S)), dim3(256), 0, st, p, spans, n_spans, ramp_n,
                       U);
    DP_HIP(hipGetLastError());
}

// p.checks was zeroed by the validation kernel
void launch_checks(Plan& p, hipStream_t st) {
    const uint64_t n = p.n_docs > p.n_kept ? p.n_docs : p.n_kept;
    hipLaunchKernelGGL(k_checks, dim3(std::min<uint32_t>(blocks_for(n), 512)), dim3(256), 0, st, p);
    DP_HIP(hipGetLastError());
}

void launch_cycle_sums(Plan& p, uint64_t total, const uint64_t* next_win, uint64_t* stream_next,
                       hipStream_t st) {  // total: the cycle's slots
    const uint32_t blocks = total ? std::min<uint32_t>(blocks_for(total), 512) : 1u;
    hipLaunchKernelGGL(k_cycle_sums, dim3(blocks), dim3(256), 0, st, p, total, next_win, stream_next);
    DP_HIP(hipGetLastError());
}

void launch_zero_u32(uint32_t* a, uint64_t n, hipStream_t st) { launch_fill_u32(a, n, 0u, st); }

void launch_fill_u32(uint32_t* a, uint64_t n, uint32_t v, hipStream_t st) {
    if (n) hipLaunchKernelGGL(k_fill_u32, dim3(blocks_for(n)), dim3(256), 0, st, a, n, v);
    DP_HIP(hipGetLastError());
}

void launch_xfer(const XferList& l, hipStream_t st) {
    if (l.n == 0) return;
    if (l.n > XFER_MAX) throw HipError{hipErrorInvalidValue, "internal: transfer list"};
    for (uint32_t i = 0; i < l.n; ++i)
        if ((reinterpret_cast<uintptr_t>(l.x[i].src) | reinterpret_cast<uintptr_t>(l.x[i].dst)) & 3u)
            throw HipError{hipErrorInvalidValue, "internal: unaligned transfer"};
    hipLaunchKernelGGL(k_xfer, dim3(l.n), dim3(256), 0, st, l);
    DP_HIP(hipGetLastError());
}

}  // namespace dp
