// scan.hip — device-wide exclusive prefix sums (three passes: tile sums,
// scan of tile sums, tile scan plus offset).  Integer sums are exact and
// order-free, so the result does not depend on the launch shape.
#include "dp_common.h"

namespace dp {
namespace {

constexpr int SB = 256;          // threads per block
constexpr int SI = 8;            // items per thread
constexpr int STILE = SB * SI;   // items per tile

template <typename T>
__device__ T block_exclusive(T v, T* lds_wave, T* total) {
    // inclusive wave scan
    const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x / WAVE;
    T x = v;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        T y = __shfl_up(x, o, WAVE);
        if (lane >= o) x += y;
    }
    if (lane == WAVE - 1) lds_wave[wid] = x;
    __syncthreads();
    T before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < SB / WAVE; ++w) {
        T t = lds_wave[w];
        if (w < wid) before += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

template <typename T, typename In>
__global__ __launch_bounds__(SB) void k_tile_sums(In in, uint64_t n, T* sums) {
    __shared__ T lw[SB / WAVE];
    const uint64_t base = (uint64_t)blockIdx.x * STILE + (uint64_t)threadIdx.x * SI;
    T s = 0;
#pragma unroll
    for (int j = 0; j < SI; ++j)
        if (base + j < n) s += in(base + j);
    T tot;
    block_exclusive<T>(s, lw, &tot);
    if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

template <typename T>
__global__ __launch_bounds__(SB) void k_scan_sums(T* sums, uint64_t nb) {
    __shared__ T lw[SB / WAVE];
    T carry = 0;
    for (uint64_t c = 0; c < nb; c += SB) {
        const uint64_t i = c + threadIdx.x;
        const T v = i < nb ? sums[i] : T(0);
        T tot;
        const T ex = block_exclusive<T>(v, lw, &tot);
        if (i < nb) sums[i] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) sums[nb] = carry;
}

template <typename T, typename In>
__global__ __launch_bounds__(SB) void k_tile_scan(In in, uint64_t n, const T* sums, T* out, uint64_t nb) {
    __shared__ T lw[SB / WAVE];
    const uint64_t base = (uint64_t)blockIdx.x * STILE + (uint64_t)threadIdx.x * SI;
    T v[SI];
    T s = 0;
#pragma unroll
    for (int j = 0; j < SI; ++j) {
        v[j] = (base + j < n) ? in(base + j) : T(0);
        s += v[j];
    }
    T tot;
    T run = block_exclusive<T>(s, lw, &tot) + sums[blockIdx.x];
#pragma unroll
    for (int j = 0; j < SI; ++j) {
        if (base + j < n) out[base + j] = run;
        run += v[j];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) out[n] = sums[nb];
}

struct KeepIn {
    const uint8_t* f;
    __device__ uint32_t operator()(uint64_t i) const { return f[i] ? 1u : 0u; }
};
struct U32In {
    const uint32_t* a;
    __device__ uint32_t operator()(uint64_t i) const { return a[i]; }
};
struct LenIn {
    const uint32_t* ids;
    const uint64_t* off;
    __device__ uint64_t operator()(uint64_t i) const {
        const uint32_t d = ids[i];
        return off[d + 1] - off[d];
    }
};
// next-fit: T-token pieces of the document at order position i; with a
// stream start, only of its tokens from the start on
struct PieceCountIn {
    const uint32_t* ids;
    const uint64_t* off;
    const uint64_t* opre;           // token prefix over the order
    const uint64_t* src_doc_start;  // [S+1] first order position of each stream
    const uint16_t* source;
    const uint64_t* start;          // [S] first token of each stream, or null
    uint32_t T;
    __device__ uint32_t operator()(uint64_t i) const {
        const uint32_t d = ids[i];
        uint64_t L = off[d + 1] - off[d];
        if (start) {
            const uint32_t s = source[d];
            const uint64_t x = opre[i] - opre[src_doc_start[s]], cut = start[s];
            const uint64_t o = cut > x ? cut - x : 0;
            L = o < L ? L - o : 0;
        }
        return (uint32_t)((L + T - 1) / T);
    }
};

// wrap packing: pieces of the document at order position i = windows of its
// source's stream that it touches; x = its first token's stream position
struct WrapPieceCountIn {
    const uint32_t* ids;
    const uint64_t* off;
    const uint64_t* opre;           // token prefix over the order
    const uint64_t* src_doc_start;  // [S+1] first order position of each source
    const uint16_t* source;
    const uint64_t* start;          // [S] first token of each stream, or null
    uint32_t T;
    __device__ uint32_t operator()(uint64_t i) const {
        const uint32_t d = ids[i];
        uint64_t L = off[d + 1] - off[d];
        uint64_t x = opre[i] - opre[src_doc_start[source[d]]];
        if (start) {  // stream positions from the start on
            const uint64_t cut = start[source[d]];
            const uint64_t o = cut > x ? cut - x : 0;
            L = o < L ? L - o : 0;
            x = x + o - cut;
        }
        if (L == 0) return 0;
        return (uint32_t)((x + L - 1) / T - x / T + 1);
    }
};

template <typename T, typename In>
void scan_impl(In in, uint64_t n, T* out, void* tmp, hipStream_t st) {
    const uint64_t nb = (n + STILE - 1) / STILE;
    T* sums = static_cast<T*>(tmp);
    if (nb == 0) {
        hipLaunchKernelGGL(k_scan_sums<T>, dim3(1), dim3(SB), 0, st, sums, (uint64_t)0);
        hipLaunchKernelGGL((k_tile_scan<T, In>), dim3(1), dim3(SB), 0, st, in, (uint64_t)0,
                           (const T*)sums, out, (uint64_t)0);
        DP_HIP(hipGetLastError());
        return;
    }
    hipLaunchKernelGGL((k_tile_sums<T, In>), dim3(nb), dim3(SB), 0, st, in, n, sums);
    hipLaunchKernelGGL(k_scan_sums<T>, dim3(1), dim3(SB), 0, st, sums, nb);
    hipLaunchKernelGGL((k_tile_scan<T, In>), dim3(nb), dim3(SB), 0, st, in, n, (const T*)sums, out, nb);
    DP_HIP(hipGetLastError());
}

}  // namespace

size_t scan_temp_bytes(uint64_t n) { return ((n + STILE - 1) / STILE + 2) * sizeof(uint64_t); }

void scan_keep_u32(const uint8_t* flags, uint64_t n, uint32_t* out, void* tmp, hipStream_t st) {
    scan_impl<uint32_t>(KeepIn{flags}, n, out, tmp, st);
}
void scan_u32(const uint32_t* in, uint64_t n, uint32_t* out, void* tmp, hipStream_t st) {
    scan_impl<uint32_t>(U32In{in}, n, out, tmp, st);
}
void scan_len_u64(const uint32_t* ids, const uint64_t* offsets, uint64_t n, uint64_t* out, void* tmp,
                  hipStream_t st) {
    scan_impl<uint64_t>(LenIn{ids, offsets}, n, out, tmp, st);
}
void scan_pieces_u32(const uint32_t* ids, const uint64_t* offsets, const uint64_t* opre,
                     const uint64_t* src_doc_start, const uint16_t* source, const uint64_t* start, uint32_t T,
                     uint64_t n, uint32_t* out, void* tmp, hipStream_t st) {
    scan_impl<uint32_t>(PieceCountIn{ids, offsets, opre, src_doc_start, source, start, T}, n, out, tmp, st);
}
void scan_wrap_pieces_u32(const uint32_t* ids, const uint64_t* offsets, const uint64_t* opre,
                          const uint64_t* src_doc_start, const uint16_t* source, const uint64_t* start, uint32_t T,
                          uint64_t n, uint32_t* out, void* tmp, hipStream_t st) {
    scan_impl<uint32_t>(WrapPieceCountIn{ids, offsets, opre, src_doc_start, source, start, T}, n, out, tmp, st);
}

}  // namespace dp
