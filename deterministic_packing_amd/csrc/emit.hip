// emit.hip — emission of a rank's slice of updates [step, step+n) and the
// per-update learned-position counts.
//
// Linnet Training, Supervised fine-tuning: rows of exactly T positions with
// the rest padded, a prompted example learns only its completion, updates
// weighed by their count of learned positions; Other trainers: a position id
// 0 starts a new sequence within a row.  For a position t inside piece
// (d, o, len) placed at window offset f, u = t − f: token tokens[off[d]+o+u],
// position id u, document id d, mask 1 iff o + u ≥ prompt_len(d).  Padding:
// pad token, position 0, document −1, mask 0.
//
// One workgroup per window.  The window's piece table is staged in LDS; each
// thread produces 4 consecutive positions and writes them with one 16-byte
// store per int32 array and one 4-byte store of the mask.  In padded windows
// these stores are non-temporal: the outputs stream to HBM without taking
// cache lines (about 4 % faster, and the kernels after the batch find no dirty
// output lines to write back).  Padding-free rows keep ordinary stores: their
// edge groups are written element by element into lines that neighbouring
// windows share, and mixing the two kinds there made the rows about 10 %
// slower.  So do the digest kernels, which store the same arrays: non-temporal
// stores from their few, long-running waves made them 2-3x slower.
#include "dp_common.h"

namespace dp {
namespace {

constexpr int EB = 256;      // threads per window
constexpr int ECAP = 512;    // pieces staged in LDS

typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));  // 16-byte load, 4-byte aligned

__device__ __forceinline__ void load4(const uint32_t* src, uint32_t (&tk)[4]) {
    const u32x4a4 x = *reinterpret_cast<const u32x4a4*>(src);
    tk[0] = x.x; tk[1] = x.y; tk[2] = x.z; tk[3] = x.w;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// one group of 4 positions: 16 bytes of each int32 array, 4 mask bytes
template <bool NT>
__device__ __forceinline__ void store_group(uint32_t* tok, int32_t* pos, int32_t* doc, uint8_t* mask, uint64_t g,
                                           const uint32_t (&tk)[4], const int32_t (&ps)[4], const int32_t (&dc)[4],
                                           uint32_t mk) {
    const u32x4 t{tk[0], tk[1], tk[2], tk[3]};
    const u32x4 o{(uint32_t)ps[0], (uint32_t)ps[1], (uint32_t)ps[2], (uint32_t)ps[3]};
    const u32x4 d{(uint32_t)dc[0], (uint32_t)dc[1], (uint32_t)dc[2], (uint32_t)dc[3]};
    u32x4* const t4 = reinterpret_cast<u32x4*>(tok) + g;
    u32x4* const o4 = reinterpret_cast<u32x4*>(pos) + g;
    u32x4* const d4 = reinterpret_cast<u32x4*>(doc) + g;
    uint32_t* const m4 = reinterpret_cast<uint32_t*>(mask) + g;
    if constexpr (NT) {
        __builtin_nontemporal_store(t, t4);
        __builtin_nontemporal_store(o, o4);
        __builtin_nontemporal_store(d, d4);
        __builtin_nontemporal_store(mk, m4);
    } else {
        *t4 = t;
        *o4 = o;
        *d4 = d;
        *m4 = mk;
    }
}

struct PieceView {
    uint32_t woff, doc, mfrom;
    uint64_t src;
};

// PACKED: padding-free rows (Linnet Training, the transformers Trainer path):
// window jj of update i writes only its real positions, at row position
// a.row_start[i][jj] of update i's row (stride B/world·T), through emit_span.
template <bool PACKED>
__global__ __launch_bounds__(EB) void k_emit(Plan p, EmitArgs a) {
    __shared__ uint32_t s_woff[ECAP];
    __shared__ uint32_t s_doc[ECAP];
    __shared__ uint32_t s_mfrom[ECAP];
    __shared__ uint64_t s_src[ECAP];

    const uint32_t widx = blockIdx.x;                  // window of this launch
    uint32_t i, jj, per_i;
    const uint64_t gw = out_window(p, a, widx, &i, &jj, &per_i);
    const uint32_t q0 = p.win_first[gw], q1 = p.win_first[gw + 1];
    const uint32_t np = q1 - q0;
    const uint32_t real = p.win_real[gw];
    const bool staged = np <= ECAP;

    auto piece = [&](uint32_t q) -> PieceView {  // q relative to q0
        const uint32_t g = q0 + q;
        const uint32_t d = p.pc_doc[g], o = p.pc_off[g], f = p.pc_woff[g];
        const uint32_t pl = p.prompt_len ? p.prompt_len[d] : 0u;
        PieceView v;
        v.woff = f;
        v.doc = d;
        v.mfrom = pl > o ? f + (pl - o < 0x7FFFFFFFu ? pl - o : 0x7FFFFFFFu) : f;
        v.src = p.offsets[d] + o;
        return v;
    };
    if (staged) {
        for (uint32_t q = threadIdx.x; q < np; q += EB) {
            const PieceView v = piece(q);
            s_woff[q] = v.woff;
            s_doc[q] = v.doc;
            s_mfrom[q] = v.mfrom;
            s_src[q] = v.src;
        }
        __syncthreads();
    }
    // last piece whose window offset is ≤ t
    auto find = [&](uint32_t t) -> uint32_t {
        uint32_t lo = 0, hi = np;  // woff[lo] ≤ t < woff[hi]
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            const uint32_t w = staged ? s_woff[mid] : p.pc_woff[q0 + mid];
            if (w <= t) lo = mid;
            else hi = mid;
        }
        return lo;
    };
    auto get = [&](uint32_t q) -> PieceView {
        if (staged) return PieceView{s_woff[q], s_doc[q], s_mfrom[q], s_src[q]};
        return piece(q);
    };

    const uint32_t pad = p.pad_token;
    // Window positions [0, len) at output element out0, which need not be a
    // multiple of 4 (padding-free rows start anywhere; padded windows when T is
    // not): positions from `real` on are padding.  Store groups are 4
    // destination elements aligned to 16 bytes; the window may start mid-group
    // (`lead` elements of that group belong to the previous window), and groups
    // that straddle the window's ends are written element by element so that
    // neighbouring windows never overwrite each other.
    auto emit_span = [&](uint64_t out0, uint32_t len) {
        const uint32_t lead = (uint32_t)(out0 & 3u);
        const uint64_t base = out0 - lead;
        const uint32_t span = lead + len;
        for (uint32_t g = threadIdx.x; g < (span + 3) / 4; g += EB) {
            const int32_t tb = (int32_t)(4 * g) - (int32_t)lead;  // window position of the group's first element
            const uint32_t tf = tb < 0 ? 0u : (uint32_t)tb;       // first position inside the window
            uint32_t tk[4];
            int32_t ps[4], dc[4];
            uint32_t mk = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) { tk[e] = pad; ps[e] = 0; dc[e] = -1; }
            if (tf < real) {
                uint32_t q = find(tf);
                PieceView v = get(q);
                uint32_t next_woff = (q + 1 < np) ? (staged ? s_woff[q + 1] : p.pc_woff[q0 + q + 1]) : real;
                const uint32_t u0 = tf - v.woff;
                if (tb >= 0 && tf + 4 <= next_woff && tf + 4 <= real && v.src + u0 + 4 <= p.n_tokens) {
                    // the four positions in one piece: one 16-byte load of their tokens
                    load4(p.tokens + v.src + u0, tk);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ps[e] = (int32_t)(u0 + e);
                        dc[e] = (int32_t)v.doc;
                        mk |= (tf + e >= v.mfrom ? 1u : 0u) << (8 * e);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int32_t ts = tb + e;
                        if (ts < 0 || (uint32_t)ts >= real) continue;
                        const uint32_t t = (uint32_t)ts;
                        while (t >= next_woff && q + 1 < np) {  // next piece (contiguous up to `real`)
                            ++q;
                            v = get(q);
                            next_woff = (q + 1 < np) ? (staged ? s_woff[q + 1] : p.pc_woff[q0 + q + 1]) : real;
                        }
                        const uint32_t u = t - v.woff;
                        tk[e] = (v.src + u < p.n_tokens) ? p.tokens[v.src + u] : pad;  // guard: never read past the corpus
                        ps[e] = (int32_t)u;
                        dc[e] = (int32_t)v.doc;
                        mk |= (t >= v.mfrom ? 1u : 0u) << (8 * e);
                    }
                }
            }
            if (tb >= 0 && (uint32_t)tb + 4 <= len) {
                store_group<false>(a.tok + base, a.pos + base, a.doc + base, a.mask + base, g, tk, ps, dc, mk);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int32_t ts = tb + e;
                    if (ts < 0 || (uint32_t)ts >= len) continue;
                    const uint64_t o = base + 4 * (uint64_t)g + e;
                    a.tok[o] = tk[e];
                    a.pos[o] = ps[e];
                    a.doc[o] = dc[e];
                    a.mask[o] = (uint8_t)(mk >> (8 * e));
                }
            }
        }
    };

    if constexpr (!PACKED) {
        if (p.T % 4) {  // window widx is [widx·T, (widx+1)·T) of the outputs, not on 16-byte boundaries
            emit_span((uint64_t)widx * p.T, p.T);
            return;
        }
        // padded windows: window widx is [widx·T, (widx+1)·T) of the outputs
        const uint64_t out0 = (uint64_t)widx * p.T;
        for (uint32_t g = threadIdx.x; g < p.T / 4; g += EB) {
            const uint32_t t0 = 4 * g;
            uint32_t tk[4];
            int32_t ps[4], dc[4];
            uint32_t mk = 0;
            if (t0 >= real) {
#pragma unroll
                for (int e = 0; e < 4; ++e) { tk[e] = pad; ps[e] = 0; dc[e] = -1; }
            } else {
                uint32_t q = find(t0);
                PieceView v = get(q);
                uint32_t next_woff = (q + 1 < np) ? (staged ? s_woff[q + 1] : p.pc_woff[q0 + q + 1]) : real;
                const uint32_t u0 = t0 - v.woff;
                if (t0 + 4 <= next_woff && t0 + 4 <= real && v.src + u0 + 4 <= p.n_tokens) {
                    // the four positions in one piece: one 16-byte load of their tokens
                    load4(p.tokens + v.src + u0, tk);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ps[e] = (int32_t)(u0 + e);
                        dc[e] = (int32_t)v.doc;
                        mk |= (t0 + e >= v.mfrom ? 1u : 0u) << (8 * e);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t t = t0 + e;
                        if (t >= real) {
                            tk[e] = pad; ps[e] = 0; dc[e] = -1;
                            continue;
                        }
                        while (t >= next_woff && q + 1 < np) {  // next piece (contiguous up to `real`)
                            ++q;
                            v = get(q);
                            next_woff = (q + 1 < np) ? (staged ? s_woff[q + 1] : p.pc_woff[q0 + q + 1]) : real;
                        }
                        const uint32_t u = t - v.woff;
                        tk[e] = (v.src + u < p.n_tokens) ? p.tokens[v.src + u] : pad;  // guard: never read past the corpus
                        ps[e] = (int32_t)u;
                        dc[e] = (int32_t)v.doc;
                        mk |= (t >= v.mfrom ? 1u : 0u) << (8 * e);
                    }
                }
            }
            store_group<true>(a.tok + out0, a.pos + out0, a.doc + out0, a.mask + out0, g, tk, ps, dc, mk);
        }
    } else {
        // padding-free rows: window jj of update i from row position row_start[i][jj]
        emit_span((uint64_t)i * a.per * p.T + (uint64_t)a.row_start[(uint64_t)i * (a.per + 1) + jj], real);
    }
}

// Row starts of the padding-free rows: per update (one workgroup), an
// exclusive scan of its windows' real positions in slot order, chunk by chunk
// with a carry; then the total and the length rounded up to the bucket.
__global__ __launch_bounds__(256) void k_packed_starts(Plan p, EmitArgs a) {
    __shared__ uint64_t part[256 / WAVE];
    const uint32_t i = blockIdx.x, lane = threadIdx.x % WAVE, wid = threadIdx.x / WAVE;
    int64_t* rs = a.row_start + (uint64_t)i * (a.per + 1);
    const uint32_t per = out_per(p, a, i);  // this update's windows of the rank (≤ a.per, the row pitch)
    uint64_t carry = 0;
    for (uint32_t c0 = 0; c0 < per; c0 += 256) {
        const uint32_t jj = c0 + threadIdx.x;
        const uint64_t v = jj < per ? p.win_real[window_of(p, (uint64_t)a.step + i, a.rank * per + jj)] : 0;
        const uint64_t x = wave_incl_u64(v);  // inclusive scan in the wave (every thread takes part)
        if (lane == WAVE - 1) part[wid] = x;
        __syncthreads();
        uint64_t before = carry;
        for (uint32_t w = 0; w < wid; ++w) before += part[w];
        if (jj < per) rs[jj] = (int64_t)(before + x - v);
        uint64_t chunk = 0;
        for (uint32_t w = 0; w < 256 / WAVE; ++w) chunk += part[w];
        __syncthreads();
        carry += chunk;
    }
    for (uint32_t jj = per + threadIdx.x; jj <= a.per; jj += blockDim.x) rs[jj] = (int64_t)carry;
    if (threadIdx.x == 0) {
        const uint64_t cap = (uint64_t)per * p.T;
        uint64_t L = a.bucket > 1 ? (carry + a.bucket - 1) / a.bucket * a.bucket : carry;
        a.length[i] = (int64_t)(L < cap ? L : cap);
    }
}

// padding of each packed row between its total and its length
__global__ __launch_bounds__(256) void k_packed_pad(Plan p, EmitArgs a) {
    const uint32_t i = blockIdx.x;
    const uint64_t base = (uint64_t)i * a.per * p.T;
    const uint64_t from = (uint64_t)a.row_start[(uint64_t)i * (a.per + 1) + a.per], to = (uint64_t)a.length[i];
    for (uint64_t x = from + threadIdx.x; x < to; x += blockDim.x) {
        a.tok[base + x] = p.pad_token;
        a.pos[base + x] = 0;
        a.doc[base + x] = -1;
        a.mask[base + x] = 0;
    }
}

// learned[i] = Σ over all B slots of the window's learned positions (global,
// the same on every rank).
__global__ __launch_bounds__(256) void k_learned(Plan p, EmitArgs a) {
    __shared__ uint64_t part[256 / WAVE];
    const uint64_t b = (uint64_t)a.step + blockIdx.x;
    uint64_t s = 0;
    const uint32_t Bb = p.ramp ? p.upd_B[b] : p.B;
    for (uint32_t j = threadIdx.x; j < Bb; j += blockDim.x) s += p.win_learn[window_of(p, b, j)];
    s = wave_sum_u64(s);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x / WAVE] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t t = 0;
        for (int w = 0; w < 256 / WAVE; ++w) t += part[w];
        a.learned[blockIdx.x] = (int64_t)t;
    }
}

}  // namespace

void launch_emit(const Plan& p, const EmitArgs& a, hipStream_t st) {
    const uint64_t windows = a.n_out;
    hipLaunchKernelGGL(k_emit<false>, dim3((uint32_t)windows), dim3(EB), 0, st, p, a);
    DP_HIP(hipGetLastError());
}

void launch_emit_packed(const Plan& p, const EmitArgs& a, hipStream_t st) {
    const uint64_t windows = a.n_out;
    hipLaunchKernelGGL(k_packed_starts, dim3(a.n_steps), dim3(256), 0, st, p, a);
    hipLaunchKernelGGL(k_emit<true>, dim3((uint32_t)windows), dim3(EB), 0, st, p, a);
    hipLaunchKernelGGL(k_packed_pad, dim3(a.n_steps), dim3(256), 0, st, p, a);
    DP_HIP(hipGetLastError());
}

void launch_learned(const Plan& p, const EmitArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(k_learned, dim3(a.n_steps), dim3(256), 0, st, p, a);
    DP_HIP(hipGetLastError());
}

}  // namespace dp
