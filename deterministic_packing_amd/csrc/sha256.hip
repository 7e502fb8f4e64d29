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

struct Block {
    uint4 v[4];
};

__device__ inline Block load_block(const uint4* p) {
    Block b;
#pragma unroll
    for (int i = 0; i < 4; ++i) b.v[i] = p[i];
    return b;
}

__device__ inline void compress_block(uint32_t H[8], const Block& b) {
    uint32_t W[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        W[4 * q + 0] = bswap32(b.v[q].x);
        W[4 * q + 1] = bswap32(b.v[q].y);
        W[4 * q + 2] = bswap32(b.v[q].z);
        W[4 * q + 3] = bswap32(b.v[q].w);
    }
    sha256_compress(H, W);
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

// Placement: each wave hashes 64 windows and is pure VALU work, so a SIMD
// that holds two of them takes twice as long, and with fewer waves than SIMDs
// the kernel's time is that of the most loaded SIMD.  A workgroup is four
// independent waves (one per SIMD of its CU); the SPREAD variant reserves
// 96 KB of LDS (16 KB used per wave, the rest unused), more than half of a
// CU's 160 KB, so no CU holds two workgroups and no SIMD two waves.  Launches
// with more waves than SIMDs use the 64 KB variant instead.
constexpr uint32_t SWAVES = 4;  // waves per workgroup

template <bool SPREAD>
__global__ __launch_bounds__(64 * SWAVES) void k_window_sha(uint32_t T, EmitArgs a, uint64_t n_windows) {
    __shared__ u32x4 lds_all[(SPREAD ? 6 : 4) * 64 * SPIECES];  // 96 KB or 64 KB
    const uint32_t wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    u32x4* lds = lds_all + wave * 64 * SPIECES;                 // this wave's 16 KB
    const uint64_t w0 = ((uint64_t)blockIdx.x * SWAVES + wave) * 64;
    if (w0 >= n_windows) return;                                // whole wave past the end
    const uint32_t nblk = 13 * (T / 64);   // blocks in the record
    const uint32_t nch = (nblk + SCH - 1) / SCH;
    const uint32_t my_piece = lane % SPIECES, my_grp = lane / SPIECES;
    u32x4 stage[SLOADS];
    load_chunk(stage, a, T, w0, n_windows, 0, my_grp, my_piece);
    uint32_t H[8];
    sha256_init(H);
#pragma unroll 1
    for (uint32_t c = 0; c < nch; ++c) {
        // chunk c: registers -> LDS (swizzled); then chunk c+1 into registers
#pragma unroll
        for (uint32_t i = 0; i < SLOADS; ++i) {
            const uint32_t j = SGRP * i + my_grp;
            lds[j * SPIECES + (my_piece ^ (j % SPIECES))] = stage[i];
        }
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

// SHA-256 of an arbitrary byte string (4-byte aligned start), one lane.
__device__ void sha_bytes(const uint8_t* msg, uint64_t len, uint8_t* out) {
    uint32_t H[8];
    sha256_init(H);
    const uint64_t full = len / 64;
    for (uint64_t b = 0; b < full; ++b) {
        uint32_t W[16];
        const uint32_t* wp = reinterpret_cast<const uint32_t*>(msg + 64 * b);
#pragma unroll
        for (int i = 0; i < 16; ++i) W[i] = bswap32(wp[i]);
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

__global__ __launch_bounds__(64) void k_batch_fp(const uint8_t* digests, uint32_t B, uint32_t n, uint8_t* out) {
    const uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n) return;
    sha_bytes(digests + 32ull * B * b, 32ull * B, out + 32ull * b);
}

__global__ void k_sha_bytes(const uint8_t* msg, uint64_t len, uint8_t* out) {
    if (threadIdx.x == 0 && blockIdx.x == 0) sha_bytes(msg, len, out);
}

}  // namespace

void launch_window_sha(const Plan& p, const EmitArgs& a, hipStream_t st) {
    const uint64_t n = (uint64_t)a.n_steps * a.per;
    const uint64_t waves = (n + 63) / 64;
    const uint32_t groups = (uint32_t)((waves + SWAVES - 1) / SWAVES);
    if (waves <= 1024)  // no more waves than MI355X SIMDs (256 CUs x 4): one per SIMD
        hipLaunchKernelGGL(k_window_sha<true>, dim3(groups), dim3(64 * SWAVES), 0, st, p.T, a, n);
    else
        hipLaunchKernelGGL(k_window_sha<false>, dim3(groups), dim3(64 * SWAVES), 0, st, p.T, a, n);
    DP_HIP(hipGetLastError());
}

void launch_batch_fp(const uint8_t* digests, uint32_t B, uint32_t n_batches, uint8_t* out, hipStream_t st) {
    hipLaunchKernelGGL(k_batch_fp, dim3((n_batches + 63) / 64), dim3(64), 0, st, digests, B, n_batches, out);
    DP_HIP(hipGetLastError());
}

void launch_sha_bytes(const uint8_t* msg, uint64_t len, uint8_t* out, hipStream_t st) {
    hipLaunchKernelGGL(k_sha_bytes, dim3(1), dim3(64), 0, st, msg, len, out);
    DP_HIP(hipGetLastError());
}

}  // namespace dp
