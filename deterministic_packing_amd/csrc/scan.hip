// scan.hip — device-wide exclusive prefix sums in one pass.  Tiles take
// tickets in the order they start; a tile sums its items, publishes the sum,
// and one wavefront looks back over the preceding tiles' published sums (64
// at a time) until it meets a published inclusive prefix (decoupled
// look-back); the tile then publishes its own inclusive prefix and writes its
// items.  Status words pack state, epoch and value into 64 bits (ScanWs).  A tile only waits for tiles with lower tickets, which have started
// and never wait for it, so every wait ends.  Integer sums are exact and
// order-free, so the result does not depend on the launch shape.
#include "dp_common.h"

namespace dp {
namespace {

constexpr int SB = 256;          // threads per block
constexpr int SI = 16;           // items per thread
constexpr int STILE = SB * SI;   // items per tile

template <typename T>
__device__ T block_exclusive(T v, T* lds_wave, T* total) {
    // inclusive wave scan (every thread of the block takes part)
    const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x / WAVE;
    T x;
    if constexpr (sizeof(T) == 8) x = (T)wave_incl_u64((uint64_t)v);
    else x = (T)wave_incl_u32((uint32_t)v);
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

__device__ __forceinline__ uint64_t status_load(const uint64_t* w) {
    return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void status_store(uint64_t* w, uint64_t v) {
    __hip_atomic_store(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr uint64_t VALUE = (1ull << SCAN_VALUE_BITS) - 1;
constexpr uint32_t LOOKBACK_POLLS = 1u << 20;  // far beyond any real wait: the tiles waited for are running

template <typename T, typename In>
__global__ __launch_bounds__(SB) void k_scan(In in, uint64_t n, T* out, ScanWs ws, uint32_t epoch) {
    __shared__ T lw[SB / WAVE];
    __shared__ uint64_t s_tile, s_prefix;
    if (threadIdx.x == 0) {
        const uint32_t t = atomicAdd(ws.ticket, 1u);
        if (t == gridDim.x - 1) atomicExch(ws.ticket, 0u);  // every ticket handed out: zero for the next scan
        s_tile = t;
    }
    __syncthreads();
    const uint64_t tile = s_tile;
    const uint64_t base = tile * STILE + (uint64_t)threadIdx.x * SI;
    T v[SI];
#pragma unroll
    for (int j = 0; j < SI; ++j) v[j] = (base + j < n) ? in(base + j) : T(0);  // every load issued first
    T s = 0;
#pragma unroll
    for (int j = 0; j < SI; ++j) s += v[j];
    T tot;
    const T ex = block_exclusive<T>(s, lw, &tot);
    const uint64_t tag = (uint64_t)epoch << SCAN_VALUE_BITS;
    const uint64_t AGG = (1ull << 62) | tag, INC = (2ull << 62) | tag;
    if (threadIdx.x == 0) {
        status_store(&ws.status[tile], (tile == 0 ? INC : AGG) | ((uint64_t)tot & VALUE));
        if (tile == 0) s_prefix = 0;
    }
    if (tile > 0 && threadIdx.x < WAVE) {
        // lane l reads tile j − l; lanes up to the first (nearest) tile with an
        // inclusive prefix add their values: sums, then that prefix
        const uint32_t lane = threadIdx.x;
        uint64_t prefix = 0;
        int64_t j = (int64_t)tile - 1;
        uint32_t polls = 0;
        while (true) {
            const int64_t q = j - (int64_t)lane;
            const uint64_t w = q >= 0 ? status_load(&ws.status[q]) : INC;  // before tile 0: a prefix of 0
            const uint64_t state = w & ~VALUE;
            if (!__all(state == AGG || state == INC)) {
                if (++polls > LOOKBACK_POLLS) {
                    if (lane == 0) atomicOr(ws.err, ERR_INTERNAL);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                continue;
            }
            const uint64_t inc = __ballot(state == INC);
            const uint32_t k = inc ? (uint32_t)__builtin_ctzll(inc) : WAVE;
            prefix += wave_sum_u64(lane <= k ? (w & VALUE) : 0);
            if (inc) break;
            j -= WAVE;
        }
        if (lane == 0) {
            status_store(&ws.status[tile], INC | ((prefix + (uint64_t)tot) & VALUE));
            s_prefix = prefix;
        }
    }
    __syncthreads();
    T run = (T)s_prefix + ex;
#pragma unroll
    for (int j = 0; j < SI; ++j) {
        if (base + j < n) out[base + j] = run;
        run += v[j];
    }
    if (tile == gridDim.x - 1 && threadIdx.x == 0) out[n] = (T)s_prefix + tot;
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
void scan_impl(In in, uint64_t n, T* out, const ScanWs& ws, hipStream_t st) {
    const uint64_t tiles = n ? (n + STILE - 1) / STILE : 1;  // n = 0: one tile writes out[0] = 0
    uint32_t epoch = ++*ws.epoch;  // a new epoch for every scan of this workspace
    if (epoch >= (1u << (62 - SCAN_VALUE_BITS))) {  // wrapped: no stale status word may carry a reused epoch
        launch_zero_u32(ws.ticket, ws.words, st);
        epoch = *ws.epoch = 1;
    }
    hipLaunchKernelGGL((k_scan<T, In>), dim3((uint32_t)tiles), dim3(SB), 0, st, in, n, out, ws, epoch);
    DP_HIP(hipGetLastError());
}

}  // namespace

uint64_t scan_ws_tiles(uint64_t n_max) { return (n_max + STILE - 1) / STILE + 1; }

size_t scan_ws_bytes(uint64_t n_max) { return 8 + 8 * scan_ws_tiles(n_max); }  // [ticket, pad][status × tiles]

ScanWs scan_ws_at(void* base, uint64_t n_max, uint32_t* err, uint32_t* host_epoch) {
    ScanWs ws{};
    ws.ticket = static_cast<uint32_t*>(base);
    ws.status = base ? reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(base) + 8) : nullptr;
    ws.err = err;
    ws.epoch = host_epoch;
    ws.words = scan_ws_bytes(n_max) / 4;
    return ws;
}

void scan_keep_u32(const uint8_t* flags, uint64_t n, uint32_t* out, const ScanWs& ws, hipStream_t st) {
    scan_impl<uint32_t>(KeepIn{flags}, n, out, ws, st);
}
void scan_u32(const uint32_t* in, uint64_t n, uint32_t* out, const ScanWs& ws, hipStream_t st) {
    scan_impl<uint32_t>(U32In{in}, n, out, ws, st);
}
void scan_len_u64(const uint32_t* ids, const uint64_t* offsets, uint64_t n, uint64_t* out, const ScanWs& ws,
                  hipStream_t st) {
    scan_impl<uint64_t>(LenIn{ids, offsets}, n, out, ws, st);
}
void scan_pieces_u32(const uint32_t* ids, const uint64_t* offsets, const uint64_t* opre,
                     const uint64_t* src_doc_start, const uint16_t* source, const uint64_t* start, uint32_t T,
                     uint64_t n, uint32_t* out, const ScanWs& ws, hipStream_t st) {
    scan_impl<uint32_t>(PieceCountIn{ids, offsets, opre, src_doc_start, source, start, T}, n, out, ws, st);
}
void scan_wrap_pieces_u32(const uint32_t* ids, const uint64_t* offsets, const uint64_t* opre,
                          const uint64_t* src_doc_start, const uint16_t* source, const uint64_t* start, uint32_t T,
                          uint64_t n, uint32_t* out, const ScanWs& ws, hipStream_t st) {
    scan_impl<uint32_t>(WrapPieceCountIn{ids, offsets, opre, src_doc_start, source, start, T}, n, out, ws, st);
}

}  // namespace dp
