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

__device__ inline void load_block_words(const uint32_t* w, uint32_t W[16]) {
    const uint4* v = reinterpret_cast<const uint4*>(w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 x = v[i];
        W[4 * i + 0] = bswap32(x.x);
        W[4 * i + 1] = bswap32(x.y);
        W[4 * i + 2] = bswap32(x.z);
        W[4 * i + 3] = bswap32(x.w);
    }
}

__device__ inline void hash_stream(uint32_t H[8], const uint32_t* words, uint32_t n_words) {
    for (uint32_t b = 0; b < n_words; b += 16) {
        uint32_t W[16];
        load_block_words(words + b, W);
        sha256_compress(H, W);
    }
}

__device__ inline void store_digest(const uint32_t H[8], uint8_t* out) {
    uint4* o = reinterpret_cast<uint4*>(out);
    o[0] = make_uint4(bswap32(H[0]), bswap32(H[1]), bswap32(H[2]), bswap32(H[3]));
    o[1] = make_uint4(bswap32(H[4]), bswap32(H[5]), bswap32(H[6]), bswap32(H[7]));
}

__global__ __launch_bounds__(64) void k_window_sha(uint32_t T, EmitArgs a, uint64_t n_windows) {
    const uint64_t w = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (w >= n_windows) return;
    const uint64_t base = w * T;
    uint32_t H[8];
    sha256_init(H);
    hash_stream(H, a.tok + base, T);
    hash_stream(H, reinterpret_cast<const uint32_t*>(a.pos + base), T);
    hash_stream(H, reinterpret_cast<const uint32_t*>(a.doc + base), T);
    hash_stream(H, reinterpret_cast<const uint32_t*>(a.mask + base), T / 4);
    // 13·T bytes is a multiple of 64 (T % 64 == 0): one padding block
    uint32_t W[16];
    W[0] = 0x80000000u;
#pragma unroll
    for (int i = 1; i < 14; ++i) W[i] = 0;
    const uint64_t bits = 13ull * T * 8ull;
    W[14] = (uint32_t)(bits >> 32);
    W[15] = (uint32_t)bits;
    sha256_compress(H, W);
    store_digest(H, a.digests + 32 * w);
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
    hipLaunchKernelGGL(k_window_sha, dim3((uint32_t)((n + 63) / 64)), dim3(64), 0, st, p.T, a, n);
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
