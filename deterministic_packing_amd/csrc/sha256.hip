// sha256.hip — window digests, batch fingerprints and byte-string digests.
//
// Zephon blog post, resume of a 16-GPU run on 8/32/64 GPUs: the SHA-256 of
// every global batch matches the original run byte for byte.  Here a window's
// digest is the SHA-256 (FIPS 180-4) of its 13·T-byte record
// tok ‖ pos ‖ doc ‖ mask (little-endian words, mask as bytes), and a batch's
// fingerprint is the SHA-256 of its B window digests in slot order, so every
// rank digests its own slice.
//
// One lane per window: SHA-256 is a serial chain per message, so the
// parallelism is across windows; the work is integer VALU (alignbit, bitop3,
// add3) with 64-byte loads per block.
#include "dp_common.h"

namespace dp {
namespace {

__device__ inline void store_digest(const uint32_t H[8], uint8_t* out) {
    uint4* o = reinterpret_cast<uint4*>(out);
    o[0] = make_uint4(bswap32(H[0]), bswap32(H[1]), bswap32(H[2]), bswap32(H[3]));
    o[1] = make_uint4(bswap32(H[4]), bswap32(H[5]), bswap32(H[6]), bswap32(H[7]));
}

// One lane per window (64 windows per wave, one wave per workgroup).  The
// record is T words of tok, T of pos, T of doc, then T/4 words of mask bytes;
// with T a multiple of 64 every 64-byte block lies in one array, and so does
// every chunk of 4 blocks (256 B) (T/16 is a multiple of 4), except a final
// partial chunk.
//
// Memory: a lane reading only its own window touches 64 windows 16 KB apart
// per instruction, which HBM serves at one row activation per 128-byte line.
// Instead the wave loads the next 256-byte chunk of its 64 windows
// cooperatively — 16 lanes read one window's 256 contiguous bytes, so each
// instruction covers four whole chunks — and keeps it in registers while the
// current chunk is hashed; then it transposes it through LDS: piece p (16 B)
// of window j sits in slot p ^ (j mod 16) of j's 256-byte row, so the lanes of
// a ds_read_b128 pass hit distinct banks.
constexpr uint32_t SCH = 4;              // blocks per chunk
constexpr uint32_t SPIECES = SCH * 4;    // 16-byte pieces per chunk per window
constexpr uint32_t SGRP = 64 / SPIECES;  // windows per load instruction
constexpr uint32_t SLOADS = 64 / SGRP;   // load instructions per chunk
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in VGPRs
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));  // 16-byte load, 4-byte aligned

// Loads chunk c of windows w0 .. w0+63 for this lane's (group, piece).  Lanes
// past the last window or past the record's last block load a clamped, valid
// address instead (their values are never hashed), so every load is
// unconditional and `stage` stays in registers.
__device__ __forceinline__ void load_chunk(u32x4 (&stage)[SLOADS], const EmitArgs& a, uint32_t T, uint64_t w0,
                                           uint64_t n_windows, uint32_t c, uint32_t my_grp, uint32_t my_piece) {
    const uint32_t per = T / 16;                         // blocks per int32 array
    const uint32_t blk0 = c * SCH;                       // uniform
    const uint32_t s = blk0 < 3 * per ? blk0 / per : 3;  // array of this chunk (uniform)
    const uint32_t nj = s < 3 ? per : T / 64;            // blocks in that array
    uint32_t j = blk0 - s * per + my_piece / 4;          // this piece's block in the array
    if (j >= nj) j = nj - 1;                             // partial last chunk
    const uint8_t* arr = s == 0 ? reinterpret_cast<const uint8_t*>(a.tok)
                       : s == 1 ? reinterpret_cast<const uint8_t*>(a.pos)
                       : s == 2 ? reinterpret_cast<const uint8_t*>(a.doc)
                                : a.mask;
    const uint64_t wbytes = (s < 3 ? 4ull : 1ull) * T;  // bytes per window in that array
    const uint8_t* piece = arr + 64ull * j + 16ull * (my_piece & 3);
#pragma unroll
    for (uint32_t i = 0; i < SLOADS; ++i) {
        uint64_t win = w0 + SGRP * i + my_grp;
        if (win >= n_windows) win = n_windows - 1;
        stage[i] = *reinterpret_cast<const u32x4*>(piece + win * wbytes);
    }
}

// Placement: each hashing wave digests 64 windows and is pure VALU work, so a
// SIMD that holds two of them takes twice as long.  The emission-and-digest
// kernel below therefore gives each SIMD of a CU exactly one hashing wave:
// its workgroups reserve 96 KB of LDS (16 KB used per hashing wave, the rest
// unused), more than half of a CU's 160 KB, so no CU holds two workgroups.

// Waits until the emitting wave of the same workgroup has published at least
// `need` record blocks of its 64 windows (workgroup-scope acquire).  The
// emitting wave never waits on anything, so the wait ends; the spin limit is
// a safety net only: the wave then flags ERR_INTERNAL in err (the batch error
// word that pack_status reports) and goes on, so every wave still exits and
// the kernel completes.  With the test option TEST_WAIT_GIVE_UP the wait asks
// for a count no wave publishes and gives up after one poll.
__device__ __forceinline__ void wait_progress(const uint32_t* prog, uint32_t need, uint32_t* err, uint32_t opts) {
    const bool give_up = (opts & TEST_WAIT_GIVE_UP) != 0;
    const uint32_t target = give_up ? 0xFFFFFFFFu : need;
    const uint32_t limit = give_up ? 1u : (1u << 24);
    uint32_t spins = 0;
    while (__hip_atomic_load(prog, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        if (++spins >= limit) {
            atomicOr(err, ERR_INTERNAL);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// Hashes windows w0 .. w0+63 of the outputs (one lane per window), reading
// each 256-byte chunk cooperatively and transposing it through this wave's
// 16 KB of LDS.  Chunk c is read only once the emitting wave has published
// its blocks in prog.
__device__ __forceinline__ void hash_outputs(uint32_t T, const EmitArgs& a, uint64_t n_windows, uint64_t w0,
                                             uint32_t lane, u32x4* lds, const uint32_t* prog, uint32_t* err,
                                             uint32_t opts) {
    const uint32_t nblk = 13 * (T / 64);   // blocks in the record
    const uint32_t nch = (nblk + SCH - 1) / SCH;
    const uint32_t my_piece = lane % SPIECES, my_grp = lane / SPIECES;
    u32x4 stage[SLOADS];
    wait_progress(prog, SCH < nblk ? SCH : nblk, err, opts);
    load_chunk(stage, a, T, w0, n_windows, 0, my_grp, my_piece);
    uint32_t H[8];
    sha256_init(H);
#pragma unroll 1
    for (uint32_t c = 0; c < nch; ++c) {
        // chunk c: registers -> LDS (swizzled); then chunk c+1 into registers
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();  // the previous chunk's LDS reads are done
#pragma unroll
        for (uint32_t i = 0; i < SLOADS; ++i) {
            const uint32_t j = SGRP * i + my_grp;
            lds[j * SPIECES + (my_piece ^ (j % SPIECES))] = stage[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (c + 1 < nch) wait_progress(prog, (c + 2) * SCH < nblk ? (c + 2) * SCH : nblk, err, opts);
        // the last iteration reloads its own chunk (harmless) so the loop has no branch around the loads
        load_chunk(stage, a, T, w0, n_windows, c + 1 < nch ? c + 1 : c, my_grp, my_piece);
        const uint32_t nb = (c + 1) * SCH <= nblk ? SCH : nblk - c * SCH;
#pragma unroll 1
        for (uint32_t b = 0; b < nb; ++b) {
            uint32_t W[16];
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q) {
                const u32x4 v = lds[lane * SPIECES + ((4 * b + q) ^ (lane % SPIECES))];
                W[4 * q + 0] = bswap32(v.x);
                W[4 * q + 1] = bswap32(v.y);
                W[4 * q + 2] = bswap32(v.z);
                W[4 * q + 3] = bswap32(v.w);
            }
            sha256_compress(H, W);
        }
    }
    // 13·T bytes is a multiple of 64: one padding block
    uint32_t W[16];
    W[0] = 0x80000000u;
#pragma unroll
    for (int i = 1; i < 14; ++i) W[i] = 0;
    const uint64_t bits = 13ull * T * 8ull;
    W[14] = (uint32_t)(bits >> 32);
    W[15] = (uint32_t)bits;
    sha256_compress(H, W);
    if (w0 + lane < n_windows) store_digest(H, a.digests + 32 * (w0 + lane));
}

// ---------------------------------------------------------------- emission beside the digest
// With digests requested, pack_batch runs one kernel whose workgroups pair
// four emitting waves with four hashing waves (one of each per SIMD).
// Emitting wave e writes the record of its 64 windows (one lane per window)
// block by block in record order and publishes, in LDS, how many blocks are
// complete; hashing wave e digests the same windows from the outputs
// (hash_outputs), reading a chunk only once it is published.  Emission is
// memory traffic and a little integer work, so it hides under the hashing
// waves' SHA-256 chains, the step's longest serial dependency, instead of
// running as a kernel of its own before them.  It serves launches of 513 to
// 1,024 waves (one hashing wave per SIMD); smaller launches use the ring
// pairs and larger ones k_emit_digest below.
//
// Piece view (plan array pc_emit, written with the window offsets): position
// t of piece q holds token base_q + t, position id t − f_q, document id d_q,
// and learns iff t ≥ mfrom_q.  After the window's real positions comes a
// padding piece (pad token, position 0, document −1, mask 0), then a piece
// that never starts.
constexpr uint32_t NEVER = 0x7FFFFFFFu;  // above every window position, positive as int32
constexpr uint32_t FWAVES = 8;           // waves per workgroup: 4 hashing, 4 emitting

struct EPiece {
    uint64_t base;   // token index of window position 0
    uint32_t woff;   // first window position
    uint32_t doc;    // document id (0xFFFFFFFF = −1 for padding)
    uint32_t mfrom;  // first learned window position (NEVER for padding)
    uint32_t pm;     // all ones for a real piece, 0 for padding
};

__device__ __forceinline__ EPiece fetch_piece(const Plan& p, uint32_t q, uint32_t q1, uint32_t real) {
    const uint32_t qq = q < q1 ? q : q1 - 1;  // every window holds at least one piece
    const uint4 e = p.pc_emit[qq];
    const uint32_t wo = p.pc_woff[qq];
    const bool in = q < q1;
    EPiece r;
    r.base = in ? ((uint64_t)e.y << 32) | e.x : 0;
    r.woff = in ? wo : (q == q1 ? real : NEVER);
    r.doc = in ? e.z : 0xFFFFFFFFu;
    r.mfrom = in ? e.w : NEVER;
    r.pm = in ? 0xFFFFFFFFu : 0u;
    return r;
}

// The piece holding the current position, the next one, and a prefetched third.
struct ECursor {
    EPiece cur, nxt, nn;
    uint32_t qn;  // piece index of nn
    __device__ __forceinline__ void restart(const Plan& p, uint32_t q0, uint32_t q1, uint32_t real) {
        cur = fetch_piece(p, q0, q1, real);
        nxt = fetch_piece(p, q0 + 1, q1, real);
        nn = fetch_piece(p, q0 + 2, q1, real);
        qn = q0 + 2;
    }
    __device__ __forceinline__ void seek(const Plan& p, uint32_t t, uint32_t q1, uint32_t real) {
        while (t >= nxt.woff) {
            cur = nxt;
            nxt = nn;
            ++qn;
            nn = fetch_piece(p, qn, q1, real);
        }
    }
};

__device__ __forceinline__ bool wave_any(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0; }
__device__ __forceinline__ int clamp4(int x) { return x < 0 ? 0 : (x > 4 ? 4 : x); }
// little-endian mask word whose bytes j..3 are 1 (j in [0, 4])
__device__ __forceinline__ uint32_t ones_le(int j) { return (uint32_t)(0x01010101ull << (8 * j)); }

__device__ __forceinline__ void load16(uint32_t (&w)[16], const uint32_t* src) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4a4 v = reinterpret_cast<const u32x4a4*>(src)[i];
        w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
}

__device__ __forceinline__ void store16(void* dst, const uint32_t (&w)[16]) {
    u32x4* d = reinterpret_cast<u32x4*>(dst);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t u = __shfl_xor(v, o, 64);
        v = u < v ? u : v;
    }
    return v;
}

__device__ __forceinline__ void publish(uint32_t* prog, uint32_t blocks, uint32_t lane) {
    // every lane's stores complete (the explicit wait makes the release's
    // ordering of global stores before the LDS count independent of how the
    // workgroup-scope release is lowered), then the count
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_store(prog, blocks, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Emits the position ids (s = 1) or document ids (s = 2) of a lane's window
// in runs: a run writes 16 elements from the piece holding position t and
// advances t by the run's length within that piece, min(16, end − t); the
// elements past the piece end are rewritten by the next run of the same lane
// (program order), so no run selects between pieces.  The window's last
// positions, where 16 elements would cross into the next window, are written
// one by one.  Record blocks [blk0, blk0 + T/16) are published as all lanes
// complete them.
template <uint32_t s>
__device__ __forceinline__ void emit_runs(const Plan& p, const EmitArgs& a, ECursor& c, uint32_t q0, uint32_t q1,
                                          uint32_t real, uint64_t w, bool valid, uint32_t* prog, uint32_t lane,
                                          uint32_t blk0) {
    static_assert(s == 1 || s == 2, "position or document ids");
    const uint32_t T = p.T;
    c.restart(p, q0, q1, real);
    uint32_t* out = reinterpret_cast<uint32_t*>(s == 1 ? a.pos : a.doc) + w * T;
    uint32_t t = 0, published = 0, it = 0;
#pragma unroll 1
    while (wave_any(t < T)) {
        if (t < T) {
            const EPiece& P = c.cur;
            const uint32_t end = c.nxt.woff < T ? c.nxt.woff : T;  // the piece's end in the window
            const uint32_t ne = end - t < 16 ? end - t : 16;
            if (t + 16 <= T) {
                uint32_t v[16];
                if (s == 1) {
                    const uint32_t pa = (t - P.woff) & P.pm, inc = P.pm & 1u;  // padding: all 0
#pragma unroll
                    for (uint32_t e = 0; e < 16; ++e) v[e] = pa + e * inc;
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) v[e] = P.doc;
                }
                if (valid) store16(out + t, v);
            } else if (valid) {
#pragma unroll 1
                for (uint32_t e = 0; e < ne; ++e) out[t + e] = s == 1 ? (t + e - P.woff) & P.pm : P.doc;
            }
            t += ne;
            if (t < T) c.seek(p, t, q1, real);
        }
        if ((++it & 7) == 0 || !wave_any(t < T)) {
            const uint32_t done = wave_min(t) / 16;  // blocks complete in every lane
            if (done > published) {
                published = done;
                publish(prog, blk0 + done, lane);
            }
        }
    }
}

// Token runs, RG at a time: the runs' positions come from the cursor first,
// then all their loads are issued (padding reads pad16, so every load is
// unconditional and no loaded value is merged across branches), then the
// stores, in run order, so a run's tail past its piece end is rewritten by the
// next run.  Runs that cannot load 16 tokens (the window's last positions, the
// corpus end) are written element by element after the group's stores.
constexpr uint32_t RG = 4;
__device__ __forceinline__ void emit_token_runs(const Plan& p, const EmitArgs& a, ECursor& c, uint32_t q0,
                                                uint32_t q1, uint32_t real, uint64_t w, bool valid, uint32_t* prog,
                                                uint32_t lane) {
    const uint32_t T = p.T, pad = p.pad_token;
    const uint64_t n_tokens = p.n_tokens;
    c.restart(p, q0, q1, real);
    uint32_t* out = a.tok + w * T;
    uint32_t t = 0, published = 0;
#pragma unroll 1
    while (wave_any(t < T)) {
        uint32_t rt[RG], rn[RG], rpm[RG];
        uint64_t rb[RG];
        bool rv[RG];
#pragma unroll
        for (uint32_t r = 0; r < RG; ++r) {
            const bool act = t < T;
            const EPiece& P = c.cur;
            const uint32_t end = c.nxt.woff < T ? c.nxt.woff : T;  // the piece's end in the window
            const uint32_t ne = act ? (end - t < 16 ? end - t : 16) : 0;
            rt[r] = t;
            rn[r] = ne;
            rb[r] = P.base;
            rpm[r] = P.pm;
            rv[r] = act && t + 16 <= T && (!P.pm || P.base + t + 16 <= n_tokens);
            t += ne;
            if (t < T) c.seek(p, t, q1, real);
        }
        uint32_t v[RG][16];
#pragma unroll
        for (uint32_t r = 0; r < RG; ++r)
            load16(v[r], rv[r] && rpm[r] ? p.tokens + rb[r] + rt[r] : p.pad16);
        if (valid) {
#pragma unroll
            for (uint32_t r = 0; r < RG; ++r)
                if (rv[r]) store16(out + rt[r], v[r]);
#pragma unroll
            for (uint32_t r = 0; r < RG; ++r) {
                if (rv[r]) continue;
#pragma unroll 1
                for (uint32_t e = 0; e < rn[r]; ++e) {
                    const uint64_t at = rb[r] + rt[r] + e;
                    out[rt[r] + e] = rpm[r] && at < n_tokens ? p.tokens[at] : pad;
                }
            }
        }
        const uint32_t done = wave_min(t) / 16;  // blocks complete in every lane
        if (done > published) {
            published = done;
            publish(prog, done, lane);
        }
    }
}

// Emits mask block t0 .. t0+63 of a lane's window (64 bytes).  With at most
// one piece boundary in the block, the learned positions are
// [A.mfrom, B.woff) ∪ [B.mfrom, end), word by word; otherwise byte by byte.
__device__ __forceinline__ void emit_mask_block(const Plan& p, const EmitArgs& a, ECursor& c, uint32_t t0,
                                                uint32_t q1, uint32_t real, uint64_t w, bool valid) {
    c.seek(p, t0, q1, real);
    const EPiece& A = c.cur;
    const EPiece& B = c.nxt;
    uint8_t* dst = a.mask + w * p.T + t0;
    if (t0 + 64 <= c.nn.woff) {
        uint32_t v[16];
        const int ma = (int)A.mfrom - (int)t0;
        if (!wave_any(t0 + 64 > B.woff)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = ones_le(clamp4(ma - 4 * i));
        } else {
            const int wb = (int)B.woff - (int)t0, mb = (int)B.mfrom - (int)t0;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                v[i] = __builtin_amdgcn_bitop3_b32(ones_le(clamp4(ma - 4 * i)), ones_le(clamp4(wb - 4 * i)),
                                                   ones_le(clamp4(mb - 4 * i)), 0xBA);  // (x & ~y) | z
        }
        if (valid) store16(dst, v);
    } else {
#pragma unroll 1
        for (uint32_t e = 0; e < 64; ++e) {
            const uint32_t t = t0 + e;
            c.seek(p, t, q1, real);
            if (valid) dst[e] = t >= c.cur.mfrom ? 1 : 0;
        }
    }
}

// Emits windows w0 .. w0+63 (one lane per window) in record order, publishing
// the number of record blocks complete in every lane.
__device__ __forceinline__ void emit_lanes(const Plan& p, const EmitArgs& a, uint64_t n_windows, uint64_t w0,
                                           uint32_t lane, uint32_t* prog) {
    const bool valid = w0 + lane < n_windows;
    const uint64_t w = valid ? w0 + lane : n_windows - 1;  // lanes past the end mirror the last window
    uint32_t i, jj, per_i;
    const uint64_t gw = out_window(p, a, w, &i, &jj, &per_i);
    const uint32_t q0 = p.win_first[gw], q1 = p.win_first[gw + 1], real = p.win_real[gw];
    const uint32_t T = p.T, per = T / 16, nblk = 13 * (T / 64);
    ECursor c;
    emit_token_runs(p, a, c, q0, q1, real, w, valid, prog, lane);
    emit_runs<1>(p, a, c, q0, q1, real, w, valid, prog, lane, per);
    emit_runs<2>(p, a, c, q0, q1, real, w, valid, prog, lane, 2 * per);
    c.restart(p, q0, q1, real);
    uint32_t b = 3 * per;
#pragma unroll 1
    for (uint32_t t0 = 0; t0 < T; t0 += 64) {
        emit_mask_block(p, a, c, t0, q1, real, w, valid);
        ++b;
        if (b % SCH == 0 || b == nblk) publish(prog, b, lane);
    }
}

__global__ __launch_bounds__(64 * FWAVES) void k_emit_sha(Plan p, EmitArgs a, uint64_t n_windows) {
    // 64 KB of transposition buffers for the hashing waves, padded to 96 KB so
    // that a CU holds one workgroup and each SIMD one hashing wave
    __shared__ u32x4 lds_all[6 * 64 * SPIECES];
    __shared__ uint32_t prog[4];
    const uint32_t wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    if (threadIdx.x < 4) prog[threadIdx.x] = 0;
    __syncthreads();
    const uint32_t e = wave & 3;
    const uint64_t w0 = ((uint64_t)blockIdx.x * 4 + e) * 64;
    if (w0 >= n_windows) return;
    if (wave < 4)
        hash_outputs(p.T, a, n_windows, w0, lane, lds_all + e * 64 * SPIECES, prog + e, p.err_batch, p.test_opts);
    else emit_lanes(p, a, n_windows, w0, lane, prog + e);
}

// ---------------------------------------------------------------- emission and digest in one lane
// For launches of more than 1,024 waves (more windows than one wave per SIMD
// covers), each lane makes its window's record itself, 64-byte block by
// 64-byte block in record order: token ids gathered from the corpus through the
// window's pieces, position ids, document ids and loss-mask bytes computed
// from them.  It stores the blocks to the outputs and compresses them, so
// nothing is read back and no lane waits for another; without LDS and at 168
// VGPRs a SIMD holds three such waves, which keeps the SHA-256 rounds'
// dependent instructions issuing.  (With one wave per SIMD the paired kernel
// above is faster: its emitting wave runs beside the chain instead of in it.)
constexpr uint32_t GWAVES = 4;  // waves (of 64 windows) per workgroup

__device__ __forceinline__ uint32_t pos_of(const EPiece& P, uint32_t t) { return (t - P.woff) & P.pm; }

// Loads for the token block at window positions t0 .. t0+15: va gets the
// 16-token run of the piece holding t0, vb that of the next piece (the block's
// words are va below window position bw, vb from it).  Both loads are
// unconditional (a run that does not lie wholly in the corpus reads the pad
// buffer), so no loaded value crosses a branch; a lane whose block needs more
// (a third piece starts in it, or a run it needs crosses the corpus end) gets
// its words one by one instead, rarely.
__device__ __forceinline__ void issue_tokens(const Plan& p, ECursor& c, uint32_t t0, uint32_t q1, uint32_t real,
                                             uint32_t (&va)[16], uint32_t (&vb)[16], uint32_t& bw) {
    c.seek(p, t0, q1, real);
    const EPiece& A = c.cur;
    const EPiece& B = c.nxt;
    const uint64_t n = p.n_tokens;
    const uint64_t lim = n >= 16 ? n - 16 : 0;
    const bool okA = A.pm && n >= 16 && A.base + t0 <= lim;
    const bool cross = t0 + 16 > B.woff;
    const bool okB = B.pm && n >= 16 && B.base + t0 <= lim;
    const bool exact = (A.pm && !okA) || (cross && B.pm && !okB) || t0 + 16 > c.nn.woff;
    load16(va, okA ? p.tokens + A.base + t0 : p.pad16);
    load16(vb, cross && okB ? p.tokens + B.base + t0 : p.pad16);
    bw = B.woff;
    if (wave_any(exact) && exact) {
        ECursor x = c;
#pragma unroll
        for (uint32_t e = 0; e < 16; ++e) {
            const uint32_t t = t0 + e;
            x.seek(p, t, q1, real);
            va[e] = x.cur.pm ? p.tokens[x.cur.base + t] : p.pad_token;
        }
        bw = NEVER;
    }
}

// Position ids (S = 1) or document ids (S = 2) of window positions t0 .. t0+15.
template <uint32_t S>
__device__ __forceinline__ void id_block(const Plan& p, ECursor& c, uint32_t t0, uint32_t q1, uint32_t real,
                                         uint32_t (&W)[16]) {
    c.seek(p, t0, q1, real);
    const EPiece& A = c.cur;
    const EPiece& B = c.nxt;
    if (!wave_any(t0 + 16 > c.nn.woff)) {  // at most one piece boundary in every lane's block
#pragma unroll
        for (uint32_t e = 0; e < 16; ++e) {
            const uint32_t t = t0 + e;
            const bool inB = t >= B.woff;
            W[e] = S == 1 ? (inB ? pos_of(B, t) : pos_of(A, t)) : (inB ? B.doc : A.doc);
        }
    } else {
        ECursor x = c;
#pragma unroll
        for (uint32_t e = 0; e < 16; ++e) {
            const uint32_t t = t0 + e;
            x.seek(p, t, q1, real);
            W[e] = S == 1 ? pos_of(x.cur, t) : x.cur.doc;
        }
    }
}

// Loss-mask bytes of window positions t0 .. t0+63 as 16 little-endian words:
// position t learns iff t is at or past the first learned position of the
// piece holding it.  With at most one boundary (A to B) in the block, the
// learned positions are [A.mfrom, B.woff) and [B.mfrom, ...), word by word.
__device__ __forceinline__ void mask_block(const Plan& p, ECursor& c, uint32_t t0, uint32_t q1, uint32_t real,
                                           uint32_t (&W)[16]) {
    c.seek(p, t0, q1, real);
    const EPiece& A = c.cur;
    const EPiece& B = c.nxt;
    if (!wave_any(t0 + 64 > c.nn.woff)) {
        const int ma = (int)A.mfrom - (int)t0, wb = (int)B.woff - (int)t0, mb = (int)B.mfrom - (int)t0;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            W[i] = __builtin_amdgcn_bitop3_b32(ones_le(clamp4(ma - 4 * i)), ones_le(clamp4(wb - 4 * i)),
                                               ones_le(clamp4(mb - 4 * i)), 0xBA);  // (x & ~y) | z
    } else {
        ECursor x = c;
#pragma unroll 1
        for (uint32_t i = 0; i < 16; ++i) {
            uint32_t w = 0;
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) {
                const uint32_t t = t0 + 4 * i + k;
                x.seek(p, t, q1, real);
                w |= (t >= x.cur.mfrom ? 1u : 0u) << (8 * k);
            }
            W[i] = w;
        }
    }
}

// Compresses the block from a byte-swapped copy, so W stays as stored.
__device__ __forceinline__ void compress_copy(uint32_t H[8], const uint32_t (&W)[16]) {
    uint32_t B[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) B[e] = bswap32(W[e]);
    sha256_compress(H, B);
}

__global__ __launch_bounds__(64 * GWAVES) __attribute__((amdgpu_waves_per_eu(3)))
void k_emit_digest(Plan p, EmitArgs a, uint64_t n_windows) {
    const uint32_t wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const uint64_t w0 = ((uint64_t)blockIdx.x * GWAVES + wave) * 64;
    if (w0 >= n_windows) return;  // whole wave past the end
    const bool valid = w0 + lane < n_windows;
    const uint64_t w = valid ? w0 + lane : n_windows - 1;  // lanes past the end mirror the last window
    uint32_t i_, jj_, per_;
    const uint64_t gw = out_window(p, a, w, &i_, &jj_, &per_);
    const uint32_t q0 = p.win_first[gw], q1 = p.win_first[gw + 1], real = p.win_real[gw];
    const uint32_t T = p.T;  // a multiple of 64 here: each array is a whole number of 128-byte lines
    if (q1 <= q0 || real > T) {  // every window holds a piece and at most T positions (else a library bug)
        atomicOr(p.err_batch, ERR_INTERNAL);
        return;
    }
    uint32_t H[8];
    sha256_init(H);
    ECursor c;
    // Blocks go in pairs, the two halves of a 128-byte line of their array:
    // the pair is stored with eight 16-byte stores in a row (no line left
    // half-written in L2 for a whole compression), each block compressed from
    // a byte-swapped copy; every loop takes two blocks per turn, so no block's
    // words are copied to other registers at a turn's end.
    auto store_pair = [&](uint8_t* dst, const uint32_t (&W0)[16], const uint32_t (&W1)[16]) {
        if (valid) {
            store16(dst, W0);
            store16(dst + 64, W1);
        }
    };
    const uint32_t nb = T / 16;  // blocks of tok, pos and doc: a multiple of 4
    // token ids: two prefetch buffers in turn, each block's runs loaded before the previous block is compressed
    uint32_t va0[16], vb0[16], bw0, va1[16], vb1[16], bw1;
    c.restart(p, q0, q1, real);
    issue_tokens(p, c, 0, q1, real, va0, vb0, bw0);
    uint8_t* const tok = reinterpret_cast<uint8_t*>(a.tok + w * T);
#pragma unroll 1
    for (uint32_t k = 0; k < nb; k += 2) {
        uint32_t W0[16], W1[16];
#pragma unroll
        for (uint32_t e = 0; e < 16; ++e) W0[e] = 16 * k + e >= bw0 ? vb0[e] : va0[e];
        issue_tokens(p, c, 16 * (k + 1), q1, real, va1, vb1, bw1);
        compress_copy(H, W0);
#pragma unroll
        for (uint32_t e = 0; e < 16; ++e) W1[e] = 16 * (k + 1) + e >= bw1 ? vb1[e] : va1[e];
        if (k + 2 < nb) issue_tokens(p, c, 16 * (k + 2), q1, real, va0, vb0, bw0);
        store_pair(tok + 64 * k, W0, W1);
        compress_copy(H, W1);
    }
    // position ids, document ids
    uint8_t* const pos = reinterpret_cast<uint8_t*>(a.pos + w * T);
    c.restart(p, q0, q1, real);
#pragma unroll 1
    for (uint32_t k = 0; k < nb; k += 2) {
        uint32_t W0[16], W1[16];
        id_block<1>(p, c, 16 * k, q1, real, W0);
        compress_copy(H, W0);
        id_block<1>(p, c, 16 * (k + 1), q1, real, W1);
        store_pair(pos + 64 * k, W0, W1);
        compress_copy(H, W1);
    }
    uint8_t* const doc = reinterpret_cast<uint8_t*>(a.doc + w * T);
    c.restart(p, q0, q1, real);
#pragma unroll 1
    for (uint32_t k = 0; k < nb; k += 2) {
        uint32_t W0[16], W1[16];
        id_block<2>(p, c, 16 * k, q1, real, W0);
        compress_copy(H, W0);
        id_block<2>(p, c, 16 * (k + 1), q1, real, W1);
        store_pair(doc + 64 * k, W0, W1);
        compress_copy(H, W1);
    }
    // loss mask, 64 positions per block; with an odd count the last block goes out alone
    uint8_t* const mask = a.mask + w * T;
    const uint32_t nm = T / 64;
    c.restart(p, q0, q1, real);
#pragma unroll 1
    for (uint32_t k = 0; k + 1 < nm; k += 2) {
        uint32_t W0[16], W1[16];
        mask_block(p, c, 64 * k, q1, real, W0);
        compress_copy(H, W0);
        mask_block(p, c, 64 * (k + 1), q1, real, W1);
        store_pair(mask + 64 * k, W0, W1);
        compress_copy(H, W1);
    }
    if (nm & 1) {
        uint32_t W[16];
        mask_block(p, c, 64 * (nm - 1), q1, real, W);
        if (valid) store16(mask + 64 * (nm - 1), W);
        compress_copy(H, W);
    }
    // 13·T bytes is a multiple of 64: one padding block
    uint32_t W[16];
    W[0] = 0x80000000u;
#pragma unroll
    for (int i = 1; i < 14; ++i) W[i] = 0;
    const uint64_t bits = 13ull * T * 8ull;
    W[14] = (uint32_t)(bits >> 32);
    W[15] = (uint32_t)bits;
    sha256_compress(H, W);
    if (valid) store_digest(H, a.digests + 32 * w);
}

// SHA-256 of an arbitrary byte string (4-byte aligned start), one lane.  The
// next block's words are loaded before the current block is compressed, so
// the chain does not wait on a load per block.
__device__ __forceinline__ void sha_bytes(const uint8_t* msg, uint64_t len, uint8_t* out) {
    uint32_t H[8];
    sha256_init(H);
    const uint64_t full = len / 64;
    const uint32_t* wp = reinterpret_cast<const uint32_t*>(msg);
    uint32_t nx[16];
    if (full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) nx[i] = wp[i];
    }
    for (uint64_t b = 0; b < full; ++b) {
        uint32_t W[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) W[i] = bswap32(nx[i]);
        if (b + 1 < full) {
#pragma unroll
            for (int i = 0; i < 16; ++i) nx[i] = wp[16 * (b + 1) + i];
        }
        sha256_compress(H, W);
    }
    const uint64_t rem = len - 64 * full;
    const uint32_t tail_blocks = (rem + 9 <= 64) ? 1 : 2;
    for (uint32_t tb = 0; tb < tail_blocks; ++tb) {
        uint32_t W[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t word = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint64_t at = 64ull * tb + 4 * i + k;  // byte index within the tail
                uint32_t byte = 0;
                if (at < rem) byte = msg[64 * full + at];
                else if (at == rem) byte = 0x80;
                word = (word << 8) | byte;
            }
            W[i] = word;
        }
        if (tb == tail_blocks - 1) {
            const uint64_t bits = len * 8ull;
            W[14] = (uint32_t)(bits >> 32);
            W[15] = (uint32_t)bits;
        }
        sha256_compress(H, W);
    }
    uint8_t* o = out;
    for (int i = 0; i < 8; ++i) {
        o[4 * i + 0] = (uint8_t)(H[i] >> 24);
        o[4 * i + 1] = (uint8_t)(H[i] >> 16);
        o[4 * i + 2] = (uint8_t)(H[i] >> 8);
        o[4 * i + 3] = (uint8_t)H[i];
    }
}

// ---------------------------------------------------------------- emission with the schedule beside the rounds
// For launches of at most 1,024 waves (a hashing wave's chain is then the
// step's critical path): pairs of waves.  The emitting wave of a pair makes
// its 64 windows' records itself, block by block (as k_emit_digest does),
// stores them, and for each block also expands the SHA-256 message schedule
// and writes its 64 words, round constants added, to a ring of RING slots in
// LDS; the hashing wave runs only the rounds, reading each round's word from
// its row, and hands the slot back.  A lone wavefront runs the rounds alone
// at about 1.7 µs per 64-byte block against 2.5 µs for the whole compression
// (the message schedule is a third of it), and neither wave reads a record
// back.  PAIRS = 1 or 2: one workgroup per CU (it reserves more than half of
// the LDS), waves 0 .. PAIRS−1 hash, the next PAIRS emit, so with waves placed
// on SIMDs in turn every wave has a SIMD of its own (launches of at most 256
// and 512 waves).  (Four pairs per CU, one hashing and one emitting wave per
// SIMD, measured slower than the paired kernel above.)
constexpr uint32_t RING = 2;          // schedule slots per pair
constexpr uint32_t RING_ROW = 65;     // words per lane's row (64, padded: no bank conflicts)
constexpr uint32_t RING_SLOT = 64 * RING_ROW;

__device__ __forceinline__ void publish_count(uint32_t* c, uint32_t v) {
    __hip_atomic_store(c, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The message schedule of block X (16 big-endian words), round constants added, into row[0..63].
__device__ __forceinline__ void schedule_row(uint32_t (&X)[16], uint32_t* row) {
#pragma unroll
    for (int t = 0; t < 64; ++t) {
        uint32_t w;
        if (t < 16) {
            w = X[t];
        } else {
            const uint32_t w15 = X[(t + 1) & 15], w2 = X[(t + 14) & 15];
            const uint32_t s0 = __builtin_amdgcn_bitop3_b32(rotr32(w15, 7), rotr32(w15, 18), w15 >> 3, 0x96);
            const uint32_t s1 = __builtin_amdgcn_bitop3_b32(rotr32(w2, 17), rotr32(w2, 19), w2 >> 10, 0x96);
            w = X[t & 15] + s0 + X[(t + 9) & 15] + s1;
            X[t & 15] = w;
        }
        row[t] = w + sha_k(t);
    }
}

__device__ __forceinline__ void rounds_from_row(uint32_t H[8], const uint32_t* row) {
    uint32_t a = H[0], b = H[1], c = H[2], d = H[3], e = H[4], f = H[5], g = H[6], h = H[7];
#pragma unroll
    for (int t = 0; t < 64; ++t) {
        const uint32_t S1 = __builtin_amdgcn_bitop3_b32(rotr32(e, 6), rotr32(e, 11), rotr32(e, 25), 0x96);
        const uint32_t ch = __builtin_amdgcn_bitop3_b32(e, f, g, 0xCA);
        const uint32_t T1 = h + row[t] + ch + S1;
        const uint32_t S0 = __builtin_amdgcn_bitop3_b32(rotr32(a, 2), rotr32(a, 13), rotr32(a, 22), 0x96);
        const uint32_t mj = __builtin_amdgcn_bitop3_b32(a, b, c, 0xE8);
        h = g; g = f; f = e; e = d + T1;
        d = c; c = b; b = a; a = T1 + S0 + mj;
    }
    H[0] += a; H[1] += b; H[2] += c; H[3] += d;
    H[4] += e; H[5] += f; H[6] += g; H[7] += h;
}

// Hashing wave of a pair: block b's row is ready once prod ≥ b + 1; the slot
// goes back (cons = b + 1) when the rounds have read it.
__device__ __forceinline__ void ring_hash(const EmitArgs& a, uint64_t n_windows, uint64_t w0, uint32_t lane,
                                          uint32_t nblk, const uint32_t* ring, uint32_t* prod, uint32_t* cons,
                                          uint32_t* err, uint32_t opts) {
    uint32_t H[8];
    sha256_init(H);
#pragma unroll 1
    for (uint32_t b = 0; b < nblk; ++b) {
        wait_progress(prod, b + 1, err, opts);
        rounds_from_row(H, ring + (b % RING) * RING_SLOT + lane * RING_ROW);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // the row's reads are complete
        if (lane == 0) publish_count(cons, b + 1);
    }
    if (w0 + lane < n_windows) store_digest(H, a.digests + 32 * (w0 + lane));
}

// Emitting wave of a pair: the records of windows w0 .. w0+63 (one lane each),
// stored like k_emit_digest's, each block's schedule into the ring.
__device__ __forceinline__ void ring_emit(const Plan& p, const EmitArgs& a, uint64_t n_windows, uint64_t w0,
                                          uint32_t lane, uint32_t* ring, uint32_t* prod, const uint32_t* cons,
                                          uint32_t* err, uint32_t opts) {
    const bool valid = w0 + lane < n_windows;
    const uint64_t w = valid ? w0 + lane : n_windows - 1;  // lanes past the end mirror the last window
    uint32_t i_, jj_, per_;
    const uint64_t gw = out_window(p, a, w, &i_, &jj_, &per_);
    const uint32_t q0 = p.win_first[gw], q1 = p.win_first[gw + 1], real = p.win_real[gw];
    const uint32_t T = p.T;
    const bool ok = q1 > q0 && real <= T;  // every window holds a piece and at most T positions (else a library bug)
    if (!ok) atomicOr(p.err_batch, ERR_INTERNAL);
    uint32_t blk = 0;  // blocks handed to the hashing wave
    auto to_ring = [&](uint32_t (&X)[16]) {  // X: big-endian words of the next block
        if (blk >= RING) wait_progress(cons, blk + 1 - RING, err, opts);  // its slot is free
        schedule_row(X, ring + (blk % RING) * RING_SLOT + lane * RING_ROW);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        ++blk;
        if (lane == 0) publish_count(prod, blk);
    };
    ECursor c;
    uint32_t P[16];
    auto finish = [&](uint32_t (&W)[16], uint8_t* dst, uint32_t k, uint32_t n_arr) {
        if ((k & 1) == 0 && k + 1 < n_arr) {  // first half of a 128-byte line: stored with the second
#pragma unroll
            for (int e = 0; e < 16; ++e) P[e] = W[e];
        } else if (valid && ok) {
            if (k & 1) store16(dst - 64, P);
            store16(dst, W);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) W[e] = bswap32(W[e]);
        to_ring(W);
    };
    const uint32_t nb = T / 16;
    const uint32_t q0c = ok ? q0 : 0, q1c = ok ? q1 : 1, realc = ok ? real : 0;  // a window that fails the check is
    uint32_t va[16], vb[16], bw;                                                // made as padding (never stored)
    c.restart(p, q0c, q1c, realc);
    issue_tokens(p, c, 0, q1c, realc, va, vb, bw);
    uint8_t* const tok = reinterpret_cast<uint8_t*>(a.tok + w * T);
#pragma unroll 1
    for (uint32_t k = 0; k < nb; ++k) {
        uint32_t W[16];
#pragma unroll
        for (uint32_t e = 0; e < 16; ++e) W[e] = 16 * k + e >= bw ? vb[e] : va[e];
        if (k + 1 < nb) issue_tokens(p, c, 16 * (k + 1), q1c, realc, va, vb, bw);
        finish(W, tok + 64 * k, k, nb);
    }
    uint8_t* const pos = reinterpret_cast<uint8_t*>(a.pos + w * T);
    c.restart(p, q0c, q1c, realc);
#pragma unroll 1
    for (uint32_t k = 0; k < nb; ++k) {
        uint32_t W[16];
        id_block<1>(p, c, 16 * k, q1c, realc, W);
        finish(W, pos + 64 * k, k, nb);
    }
    uint8_t* const doc = reinterpret_cast<uint8_t*>(a.doc + w * T);
    c.restart(p, q0c, q1c, realc);
#pragma unroll 1
    for (uint32_t k = 0; k < nb; ++k) {
        uint32_t W[16];
        id_block<2>(p, c, 16 * k, q1c, realc, W);
        finish(W, doc + 64 * k, k, nb);
    }
    uint8_t* const mask = a.mask + w * T;
    c.restart(p, q0c, q1c, realc);
#pragma unroll 1
    for (uint32_t k = 0; k < T / 64; ++k) {
        uint32_t W[16];
        mask_block(p, c, 64 * k, q1c, realc, W);
        finish(W, mask + 64 * k, k, T / 64);
    }
    // 13·T bytes is a multiple of 64: one padding block
    uint32_t X[16];
    X[0] = 0x80000000u;
#pragma unroll
    for (int i = 1; i < 14; ++i) X[i] = 0;
    const uint64_t bits = 13ull * T * 8ull;
    X[14] = (uint32_t)(bits >> 32);
    X[15] = (uint32_t)bits;
    to_ring(X);
}

template <uint32_t PAIRS>
__global__ __launch_bounds__(128 * PAIRS) void k_emit_ring(Plan p, EmitArgs a, uint64_t n_windows) {
    static_assert(PAIRS <= 2, "at most two pairs: every wave on a SIMD of its own");
    // [PAIRS][RING] slots, then prod[PAIRS], cons[PAIRS], padded to 96 KB (one workgroup per CU)
    __shared__ uint32_t ring_lds[96 * 1024 / 4];
    const uint32_t wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const bool hasher = wave < PAIRS;  // waves 0 .. PAIRS−1 hash, the next PAIRS emit (wave i on SIMD i mod 4)
    const uint32_t pair = hasher ? wave : wave - PAIRS;
    uint32_t* ring = ring_lds + pair * RING * RING_SLOT;
    uint32_t* prod = ring_lds + PAIRS * RING * RING_SLOT;
    uint32_t* cons = prod + PAIRS;
    if (threadIdx.x < 2 * PAIRS) prod[threadIdx.x] = 0;
    __syncthreads();
    const uint64_t w0 = ((uint64_t)blockIdx.x * PAIRS + pair) * 64;
    if (w0 >= n_windows) return;  // both waves of the pair
    const uint32_t nblk = 13 * (p.T / 64) + 1;
    if (hasher) ring_hash(a, n_windows, w0, lane, nblk, ring, prod + pair, cons + pair, p.err_batch, p.test_opts);
    else ring_emit(p, a, n_windows, w0, lane, ring, prod + pair, cons + pair, p.err_batch, p.test_opts);
}

__global__ __launch_bounds__(64) void k_batch_fp(const uint8_t* digests, uint32_t B, uint32_t n, uint8_t* out) {
    const uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n) return;
    sha_bytes(digests + 32ull * B * b, 32ull * B, out + 32ull * b);
}

// batch b of a ramped cycle: its B_b digests, from slot slot0[step+b] − slot0[step] on
__global__ __launch_bounds__(64) void k_batch_fp_var(const uint8_t* digests, const uint64_t* slot0, uint32_t step,
                                                     uint32_t n, uint8_t* out) {
    const uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n) return;
    const uint64_t x0 = slot0[step + b] - slot0[step], x1 = slot0[step + b + 1] - slot0[step];
    sha_bytes(digests + 32ull * x0, 32ull * (x1 - x0), out + 32ull * b);
}

// SHA-256 of a byte string (4-byte aligned start) by one whole wavefront,
// for the plan digest's chains: lane l builds padded block b0 + l (64 blocks
// at a time), expands its message schedule and stores the 64 words with the
// round constants added to LDS (kw, 64 × 65 words: a padded row per lane);
// lane 0 then runs the compressions on those words, so the serial chain holds
// only the round function (about 14 of the 22 instructions of a round).
constexpr uint32_t KW_ROW = 65;

// kw: the block's 64 round words K[t] + W[t], in registers (loaded from LDS
// before the rounds, so the chain waits for LDS once per block, not per round)
__device__ __forceinline__ void sha256_compress_kw(uint32_t H[8], const uint32_t (&kw)[64]) {
    uint32_t a = H[0], b = H[1], c = H[2], d = H[3], e = H[4], f = H[5], g = H[6], h = H[7];
#pragma unroll
    for (int t = 0; t < 64; ++t) {
        const uint32_t S1 = __builtin_amdgcn_bitop3_b32(rotr32(e, 6), rotr32(e, 11), rotr32(e, 25), 0x96);
        const uint32_t ch = __builtin_amdgcn_bitop3_b32(e, f, g, 0xCA);
        const uint32_t T1 = h + kw[t] + ch + S1;
        const uint32_t S0 = __builtin_amdgcn_bitop3_b32(rotr32(a, 2), rotr32(a, 13), rotr32(a, 22), 0x96);
        const uint32_t mj = __builtin_amdgcn_bitop3_b32(a, b, c, 0xE8);
        h = g; g = f; f = e; e = d + T1;
        d = c; c = b; b = a; a = T1 + S0 + mj;
    }
    H[0] += a; H[1] += b; H[2] += c; H[3] += d;
    H[4] += e; H[5] += f; H[6] += g; H[7] += h;
}

// Word i of padded block b of an len-byte message (big-endian).
__device__ __forceinline__ uint32_t padded_word(const uint8_t* msg, uint64_t len, uint64_t nblk, uint64_t b,
                                                uint32_t i) {
    if (b == nblk - 1 && i >= 14) return i == 14 ? (uint32_t)((len * 8) >> 32) : (uint32_t)(len * 8);
    const uint64_t x = 64 * b + 4 * i;
    if (x + 4 <= len) return bswap32(reinterpret_cast<const uint32_t*>(msg)[x / 4]);
    uint32_t word = 0;
    for (uint32_t k = 0; k < 4; ++k) {
        const uint64_t at = x + k;
        word = (word << 8) | (at < len ? msg[at] : (at == len ? 0x80u : 0u));
    }
    return word;
}

__device__ __forceinline__ void sha_bytes_wave(const uint8_t* msg, uint64_t len, uint8_t* out, uint32_t* kw) {
    const uint32_t lane = lane_id();
    const uint64_t nblk = (len + 9 + 63) / 64;
    uint32_t H[8];
    sha256_init(H);
    for (uint64_t b0 = 0; b0 < nblk; b0 += WAVE) {
        const uint64_t b = b0 + lane;
        if (b < nblk) {
            uint32_t W[16];
#pragma unroll
            for (uint32_t i = 0; i < 16; ++i) W[i] = padded_word(msg, len, nblk, b, i);
            uint32_t* row = kw + lane * KW_ROW;
#pragma unroll
            for (int t = 0; t < 64; ++t) {
                uint32_t w;
                if (t < 16) {
                    w = W[t];
                } else {
                    const uint32_t w15 = W[(t + 1) & 15], w2 = W[(t + 14) & 15];
                    const uint32_t s0 = __builtin_amdgcn_bitop3_b32(rotr32(w15, 7), rotr32(w15, 18), w15 >> 3, 0x96);
                    const uint32_t s1 = __builtin_amdgcn_bitop3_b32(rotr32(w2, 17), rotr32(w2, 19), w2 >> 10, 0x96);
                    w = W[t & 15] + s0 + W[(t + 9) & 15] + s1;
                    W[t & 15] = w;
                }
                row[t] = w + sha_k(t);
            }
        }
        __syncthreads();  // one wavefront per workgroup: its schedule rows are in LDS
        if (lane == 0) {
            const uint64_t n = nblk - b0 < WAVE ? nblk - b0 : WAVE;
            for (uint64_t k = 0; k < n; ++k) {
                uint32_t r[64];
#pragma unroll
                for (int t = 0; t < 64; ++t) r[t] = kw[k * KW_ROW + t];
                sha256_compress_kw(H, r);
            }
        }
        __syncthreads();  // the rows are consumed before the next group overwrites them
    }
    if (lane == 0) store_digest(H, out);
}

__global__ __launch_bounds__(WAVE) void k_sha_bytes(const uint8_t* msg, uint64_t len, uint8_t* out) {
    __shared__ uint32_t kw[WAVE * KW_ROW];
    sha_bytes_wave(msg, len, out, kw);
}

// workgroup j (one wavefront): SHA-256 of msg[j·chunk, min((j+1)·chunk, len)) into out + 32·j
__global__ __launch_bounds__(WAVE) void k_sha_chunks(const uint8_t* msg, uint64_t len, uint32_t chunk, uint8_t* out) {
    __shared__ uint32_t kw[WAVE * KW_ROW];
    const uint64_t x0 = (uint64_t)blockIdx.x * chunk;
    const uint64_t x1 = x0 + chunk < len ? x0 + chunk : len;
    sha_bytes_wave(msg + x0, x1 - x0, out + 32ull * blockIdx.x, kw);
}

// ---------------------------------------------------------------- any window length
// T not a multiple of 64: the emission kernel writes the windows first, then
// this kernel hashes each window's record from the outputs, one lane per
// window.  Word j of the padded message (its bytes 4j .. 4j+3, big-endian for
// the compression) is element j of tok, pos, doc for j < 3T (each array is 4T
// bytes, so no word straddles two of them); from byte 12T on come the T mask
// bytes, the byte 0x80, zeros, and the message's bit length 104·T as 8
// big-endian bytes that end the last block (FIPS 180-4, section 5.1.1).
__global__ __launch_bounds__(256) void k_window_digest_any(Plan p, EmitArgs a) {
    const uint64_t w = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (w >= a.n_out) return;
    const uint64_t T = p.T, o = w * T;
    const uint32_t* tok = a.tok + o;
    const int32_t* pos = a.pos + o;
    const int32_t* doc = a.doc + o;
    const uint8_t* mask = a.mask + o;
    const uint64_t L = 13 * T;              // message bytes
    const uint64_t nb = (L + 72) / 64;      // blocks: L + 1 + 8 bytes rounded up to 64
    const uint64_t tail = 64 * nb - 8, bits = 8 * L;
    auto byte_at = [&](uint64_t i) -> uint32_t {  // byte i ≥ 12T of the padded message
        if (i < L) return mask[i - 12 * T];
        if (i == L) return 0x80u;
        if (i >= tail) return (uint32_t)(bits >> (8 * (7 - (i - tail)))) & 0xFFu;
        return 0u;
    };
    uint32_t H[8];
    sha256_init(H);
    for (uint64_t b = 0; b < nb; ++b) {
        uint32_t W[16];
#pragma unroll
        for (uint32_t e = 0; e < 16; ++e) {
            const uint64_t j = 16 * b + e;
            if (j < T) W[e] = bswap32(tok[j]);
            else if (j < 2 * T) W[e] = bswap32((uint32_t)pos[j - T]);
            else if (j < 3 * T) W[e] = bswap32((uint32_t)doc[j - 2 * T]);
            else W[e] = byte_at(4 * j) << 24 | byte_at(4 * j + 1) << 16 | byte_at(4 * j + 2) << 8 | byte_at(4 * j + 3);
        }
        sha256_compress(H, W);
    }
    store_digest(H, a.digests + 32 * w);
}

// ---------------------------------------------------------------- chunked window digests
// PACK_FLAG_DIGEST_CHUNKED: a window's digest is the SHA-256 of the SHA-256
// digests of its record's chunks of DIGEST_CHUNK bytes (the last chunk
// shorter), in record order.  The chunks are independent chains, so one lane
// hashes one chunk and a window's chunks run side by side.  The emission
// kernel writes the windows first and these kernels read each record from the
// outputs, one slice of windows [w0, w0 + nw) at a time: lane g hashes chunk
// g mod nc of window w0 + g / nc (nc chunks a window) into cd[8g .. 8g+8)
// (the final state words, which are the chunk digest's big-endian words, so
// they are the next message's words as they stand), then one lane per window
// hashes its nc chunk digests.
//
// Byte x of a record lies in tok (x < 4T), pos (x < 8T), doc (x < 12T) as
// 4-byte little-endian elements, or in mask (x ≥ 12T).
__device__ __forceinline__ const uint8_t* record_at(const EmitArgs& a, uint64_t T, uint64_t w, uint64_t x) {
    if (x < 4 * T) return reinterpret_cast<const uint8_t*>(a.tok + w * T) + x;
    if (x < 8 * T) return reinterpret_cast<const uint8_t*>(a.pos + w * T) + (x - 4 * T);
    if (x < 12 * T) return reinterpret_cast<const uint8_t*>(a.doc + w * T) + (x - 8 * T);
    return a.mask + w * T + (x - 12 * T);
}

// The padding block that ends a message of len bytes, len a multiple of 64
// (FIPS 180-4, section 5.1.1: the byte 0x80, zeros, the bit length).
__device__ __forceinline__ void final_pad_block(uint32_t H[8], uint64_t len) {
    uint32_t W[16];
    W[0] = 0x80000000u;
#pragma unroll
    for (uint32_t e = 1; e < 14; ++e) W[e] = 0u;
    W[14] = (uint32_t)((8 * len) >> 32);
    W[15] = (uint32_t)(8 * len);
    sha256_compress(H, W);
}

__device__ __forceinline__ void store_state(const uint32_t H[8], uint32_t* out) {
    uint4* o = reinterpret_cast<uint4*>(out);
    o[0] = make_uint4(H[0], H[1], H[2], H[3]);
    o[1] = make_uint4(H[4], H[5], H[6], H[7]);
}

// T a multiple of 1,024: 4T and 12T are multiples of DIGEST_CHUNK, so every
// chunk lies in one array, and every chunk length (4,096, or T mod 4,096 for
// the last mask chunk) is a multiple of 1,024.  A lane takes its chunk one
// 128-byte line (two blocks, eight 16-byte loads) at a time and loads the
// next line before compressing the current one (the last line is loaded
// twice, so every load is unconditional).
__global__ __launch_bounds__(256) void k_chunk_sha_lines(Plan p, EmitArgs a, uint64_t w0, uint64_t n_lanes,
                                                         uint32_t nc, uint32_t* cd) {
    const uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= n_lanes) return;
    const uint64_t T = p.T, w = w0 + g / nc, x0 = (uint64_t)DIGEST_CHUNK * (g % nc);
    const uint64_t len = 13 * T - x0 < DIGEST_CHUNK ? 13 * T - x0 : DIGEST_CHUNK;
    const u32x4a4* src = reinterpret_cast<const u32x4a4*>(record_at(a, T, w, x0));
    const uint32_t lines = (uint32_t)(len / 128);
    u32x4 nx[8];
#pragma unroll
    for (uint32_t e = 0; e < 8; ++e) nx[e] = src[e];
    uint32_t H[8];
    sha256_init(H);
    for (uint32_t l = 0; l < lines; ++l) {
        u32x4 cur[8];
#pragma unroll
        for (uint32_t e = 0; e < 8; ++e) cur[e] = nx[e];
        const uint32_t ln = l + 1 < lines ? l + 1 : l;
#pragma unroll
        for (uint32_t e = 0; e < 8; ++e) nx[e] = src[8 * ln + e];
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            uint32_t W[16];
#pragma unroll
            for (uint32_t e = 0; e < 4; ++e) {
                W[4 * e + 0] = bswap32(cur[4 * h + e].x);
                W[4 * e + 1] = bswap32(cur[4 * h + e].y);
                W[4 * e + 2] = bswap32(cur[4 * h + e].z);
                W[4 * e + 3] = bswap32(cur[4 * h + e].w);
            }
            sha256_compress(H, W);
        }
    }
    final_pad_block(H, len);
    store_state(H, cd + 8 * g);
}

// Any T: word j of a chunk's padded message is a whole element of tok, pos
// or doc while its 4 bytes lie before byte 12T of the record (chunk starts and
// 12T are multiples of 4, and a chunk ends at a multiple of 4 there); from
// there on the words are assembled byte by byte from mask, the byte 0x80,
// zeros and the chunk's bit length.
__global__ __launch_bounds__(256) void k_chunk_sha_any(Plan p, EmitArgs a, uint64_t w0, uint64_t n_lanes,
                                                       uint32_t nc, uint32_t* cd) {
    const uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= n_lanes) return;
    const uint64_t T = p.T, w = w0 + g / nc, x0 = (uint64_t)DIGEST_CHUNK * (g % nc);
    const uint64_t len = 13 * T - x0 < DIGEST_CHUNK ? 13 * T - x0 : DIGEST_CHUNK;
    const uint64_t nb = (len + 72) / 64, tail = 64 * nb - 8, bits = 8 * len;
    const uint8_t* mask = a.mask + w * T;
    auto byte_at = [&](uint64_t q) -> uint32_t {  // byte q of the padded chunk, x0 + q ≥ 12T when q < len
        if (q < len) return mask[x0 + q - 12 * T];
        if (q == len) return 0x80u;
        if (q >= tail) return (uint32_t)(bits >> (8 * (7 - (q - tail)))) & 0xFFu;
        return 0u;
    };
    uint32_t H[8];
    sha256_init(H);
    for (uint64_t b = 0; b < nb; ++b) {
        uint32_t W[16];
#pragma unroll
        for (uint32_t e = 0; e < 16; ++e) {
            const uint64_t q = 64 * b + 4 * e, x = x0 + q;
            if (q + 4 <= len && x + 4 <= 12 * T)
                W[e] = bswap32(*reinterpret_cast<const uint32_t*>(record_at(a, T, w, x)));
            else
                W[e] = byte_at(q) << 24 | byte_at(q + 1) << 16 | byte_at(q + 2) << 8 | byte_at(q + 3);
        }
        sha256_compress(H, W);
    }
    store_state(H, cd + 8 * g);
}

// One lane per window of the slice: SHA-256 of its nc chunk digests (8·nc
// message words, then 0x80000000, zeros and the bit length 256·nc).
__global__ __launch_bounds__(256) void k_chunk_final(EmitArgs a, uint64_t w0, uint64_t nw, uint32_t nc,
                                                     const uint32_t* cd) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nw) return;
    const uint32_t* m = cd + 8ull * nc * i;
    const uint64_t words = 8ull * nc, nb = (32ull * nc + 72) / 64, bits = 256ull * nc;
    uint32_t H[8];
    sha256_init(H);
    for (uint64_t b = 0; b < nb; ++b) {
        uint32_t W[16];
#pragma unroll
        for (uint32_t e = 0; e < 16; ++e) {
            const uint64_t j = 16 * b + e;
            W[e] = j < words ? m[j]
                   : j == words ? 0x80000000u
                   : j == 16 * nb - 2 ? (uint32_t)(bits >> 32)
                   : j == 16 * nb - 1 ? (uint32_t)bits
                   : 0u;
        }
        sha256_compress(H, W);
    }
    store_digest(H, a.digests + 32 * (w0 + i));
}

}  // namespace

// Launch shape by the number of waves of 64 windows (each a chain of 13·T/64 + 1
// compressions): at most 256, one ring pair per CU; at most 512, two (the
// hashing waves alone on their SIMDs); at most 1,024, the paired kernel with
// one hashing wave per SIMD (measured faster there than four ring pairs per
// CU, whose emitting waves share the hashing waves' SIMDs); above, each lane
// its own record (throughput-bound).
void launch_emit_sha(const Plan& p, const EmitArgs& a, hipStream_t st) {
    const uint64_t n = a.n_out;  // < 2^31 windows: at most 2^23 workgroups
    const uint64_t waves = (n + 63) / 64;
    if (!n) return;
    if (p.digest_chunked) {  // one stream: the emission, then the chunk digests slice by slice
        launch_emit(p, a, st);
        const uint64_t slice = chunk_slice_windows(p);
        for (uint64_t w0 = 0; w0 < n; w0 += slice) launch_chunk_hash(p, a, w0, n - w0 < slice ? n - w0 : slice, st);
        return;
    }
    if (p.T % 64) {  // records not made of whole 64-byte blocks per array: emission, then digests from the outputs
        launch_emit(p, a, st);
        hipLaunchKernelGGL(k_window_digest_any, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, st, p, a);
    } else if (waves <= 256)
        hipLaunchKernelGGL(k_emit_ring<1>, dim3((uint32_t)waves), dim3(128), 0, st, p, a, n);
    else if (waves <= 512)
        hipLaunchKernelGGL(k_emit_ring<2>, dim3((uint32_t)((waves + 1) / 2)), dim3(256), 0, st, p, a, n);
    else if (waves <= 1024)
        hipLaunchKernelGGL(k_emit_sha, dim3((uint32_t)((n + 255) / 256)), dim3(64 * FWAVES), 0, st, p, a, n);
    else
        hipLaunchKernelGGL(k_emit_digest, dim3((uint32_t)((waves + GWAVES - 1) / GWAVES)), dim3(64 * GWAVES), 0, st,
                           p, a, n);
    DP_HIP(hipGetLastError());
}

// Windows whose chunk digests p.chunk_cd holds at once (at least one: the
// scratch is sized at init for one window's chunks or more).
uint64_t chunk_slice_windows(const Plan& p) {
    const uint64_t slice = p.chunk_cd_words / (8 * digest_chunks(p.T));
    if (slice == 0) throw HipError{hipErrorInvalidValue, "internal: chunk digest scratch"};
    return (p.test_opts & TEST_DIGEST_SLICES) && slice > 3 ? 3 : slice;  // test option: many slices a call
}

// Chunk digests of windows [w0, w0 + nw) of a call's outputs (nw at most
// chunk_slice_windows), then their window digests into a.digests.
void launch_chunk_hash(const Plan& p, const EmitArgs& a, uint64_t w0, uint64_t nw, hipStream_t st) {
    const uint64_t nc = digest_chunks(p.T), lanes = nw * nc;
    if (!nw) return;
    if (nw > chunk_slice_windows(p)) throw HipError{hipErrorInvalidValue, "internal: chunk digest slice"};
    const dim3 grid((uint32_t)((lanes + 255) / 256));
    if (p.T % 1024 == 0)
        hipLaunchKernelGGL(k_chunk_sha_lines, grid, dim3(256), 0, st, p, a, w0, lanes, (uint32_t)nc, p.chunk_cd);
    else
        hipLaunchKernelGGL(k_chunk_sha_any, grid, dim3(256), 0, st, p, a, w0, lanes, (uint32_t)nc, p.chunk_cd);
    hipLaunchKernelGGL(k_chunk_final, dim3((uint32_t)((nw + 255) / 256)), dim3(256), 0, st, a, w0, nw, (uint32_t)nc,
                       (const uint32_t*)p.chunk_cd);
    DP_HIP(hipGetLastError());
}

void launch_batch_fp(const uint8_t* digests, uint32_t B, uint32_t n_batches, uint8_t* out, hipStream_t st) {
    hipLaunchKernelGGL(k_batch_fp, dim3((n_batches + 63) / 64), dim3(64), 0, st, digests, B, n_batches, out);
    DP_HIP(hipGetLastError());
}

void launch_batch_fp_var(const uint8_t* digests, const uint64_t* slot0, uint32_t step, uint32_t n_batches,
                         uint8_t* out, hipStream_t st) {
    hipLaunchKernelGGL(k_batch_fp_var, dim3((n_batches + 63) / 64), dim3(64), 0, st, digests, slot0, step, n_batches,
                       out);
    DP_HIP(hipGetLastError());
}

void launch_sha_chunks(const uint8_t* msg, uint64_t len, uint32_t chunk, uint8_t* out, hipStream_t st) {
    const uint64_t n = (len + chunk - 1) / chunk;  // one workgroup per chunk
    if (n) hipLaunchKernelGGL(k_sha_chunks, dim3((uint32_t)n), dim3(WAVE), 0, st, msg, len, chunk, out);
    DP_HIP(hipGetLastError());
}

void launch_sha_bytes(const uint8_t* msg, uint64_t len, uint8_t* out, hipStream_t st) {
    hipLaunchKernelGGL(k_sha_bytes, dim3(1), dim3(64), 0, st, msg, len, out);
    DP_HIP(hipGetLastError());
}

}  // namespace dp
