// api.hip — the C ABI declared in include/dpack.h: context, workspace, the
// synchronous plan (pack_init), cycles, and asynchronous batch emission.
#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "dp_common.h"
#include "dpack.h"

// The device workspace of pack_init_noalloc (see NoallocSlot below).  Host code
// never passes this name to a kernel or a copy: it uses the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[64ull << 20];

namespace {

constexpr size_t ALIGN = 256;

// One cached device workspace and one pinned host staging area per device:
// pack_destroy parks them here and the next pack_init on that device reuses
// them when large enough, so a loop of init/destroy does not pay
// hipMalloc/hipHostMalloc (and their frees) each time.
struct ArenaCache {
    std::mutex mu;
    std::vector<std::pair<void*, size_t>> per_device;  // index = device
    bool pinned;
};
ArenaCache& arena_cache(bool pinned = false) {
    static ArenaCache dev{{}, {}, false}, host{{}, {}, true};
    return pinned ? host : dev;
}

void cache_free(const ArenaCache& c, void* p) {
    if (c.pinned) (void)hipHostFree(p);
    else (void)hipFree(p);
}

void* arena_take(int dev, size_t bytes, size_t* got, bool pinned = false) {
    auto& c = arena_cache(pinned);
    std::lock_guard<std::mutex> lk(c.mu);
    if ((size_t)dev < c.per_device.size()) {
        auto& e = c.per_device[dev];
        if (e.first && e.second >= bytes) {
            void* p = e.first;
            *got = e.second;
            e = {nullptr, 0};
            return p;
        }
    }
    return nullptr;
}

void arena_give(int dev, void* ptr, size_t bytes, bool pinned = false) {
    auto& c = arena_cache(pinned);
    std::lock_guard<std::mutex> lk(c.mu);
    if ((size_t)dev >= c.per_device.size()) c.per_device.resize(dev + 1, {nullptr, 0});
    auto& e = c.per_device[dev];
    if (e.first == nullptr || e.second < bytes) {
        if (e.first) cache_free(c, e.first);
        e = {ptr, bytes};
    } else {
        cache_free(c, ptr);
    }
}

// Memory of pack_init_noalloc, for callers that cannot allocate.  The device
// workspace of such a context is carved from `scratch`, a file-scope device
// array that each GPU holds from the library's first use on it until the
// process ends; its pinned-staging role is taken by a static host buffer per
// device.  One such context may be alive per device at a time (a slot's
// in_use flag, under a mutex); its workspace keeps the previous context's
// bytes, and the plan clears what must start at zero exactly as it does in a
// workspace reused from the arena cache.
constexpr size_t NOALLOC_DEVICE_BYTES = 64ull << 20;  // 64 MiB per device
constexpr size_t NOALLOC_HOST_BYTES = 1ull << 20;     // 1 MiB of host staging per device
constexpr int NOALLOC_MAX_DEVICES = 16;

struct NoallocSlot {
    void* dev = nullptr;  // the device address of `scratch` on this device (hipGetSymbolAddress)
    bool in_use = false;
    alignas(256) uint8_t host[NOALLOC_HOST_BYTES];
};
std::mutex g_noalloc_mu;
NoallocSlot g_noalloc[NOALLOC_MAX_DEVICES];

thread_local std::string g_init_error;

uint32_t bitlen(uint64_t x) {
    uint32_t n = 0;
    while (x) {
        ++n;
        x >>= 1;
    }
    return n;
}

struct InvalError {
    std::string msg;
};

// a kernel flagged ERR_INTERNAL: a library bug or a bounded wait that gave up
struct InternalError {
    std::string msg;
};

}  // namespace

// HIP events around kernel phases, recorded on the context's stream when the
// context is made with PACK_FLAG_TIMING (every phase) or PACK_FLAG_TIMING_BATCH
// (the phases of pack_batch and pack_fingerprint); resolved in pack_get_timings.
struct PhaseTimer {
    bool on = false;
    uint32_t phases = 0;  // bit k: phase k is timed
    std::vector<hipEvent_t> pool;
    struct Pending {
        int phase;
        hipEvent_t a, b;
    };
    std::vector<Pending> pending;
    int open_phase = -1;
    hipEvent_t open_a = nullptr;
    double ms[PACK_N_PHASES] = {};
    uint64_t calls[PACK_N_PHASES] = {};

    hipEvent_t get() {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        // timestamps only: no system-scope fence (a fence writes back and invalidates the
        // caches at every phase boundary, about 10 µs each, and slows the work after it)
        hipEvent_t e;
        DP_HIP(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
        return e;
    }
    void begin(int phase, hipStream_t st) {
        if (!on || !(phases >> phase & 1u)) return;
        open_phase = phase;
        open_a = get();
        DP_HIP(hipEventRecord(open_a, st));
    }
    void end(hipStream_t st) {
        if (!on || open_phase < 0) return;
        hipEvent_t b = get();
        DP_HIP(hipEventRecord(b, st));
        pending.push_back({open_phase, open_a, b});
        open_phase = -1;
    }
    void resolve() {
        for (auto& q : pending) {
            DP_HIP(hipEventSynchronize(q.b));
            float t = 0.f;
            DP_HIP(hipEventElapsedTime(&t, q.a, q.b));
            ms[q.phase] += t;
            calls[q.phase] += 1;
            pool.push_back(q.a);
            pool.push_back(q.b);
        }
        pending.clear();
    }
    void destroy() {
        for (auto& q : pending) {
            pool.push_back(q.a);
            pool.push_back(q.b);
        }
        pending.clear();
        if (open_phase >= 0) pool.push_back(open_a);
        for (hipEvent_t e : pool) (void)hipEventDestroy(e);
        pool.clear();
    }
};

struct pack_ctx {
    pack_config cfg{};
    PhaseTimer timer;
    std::vector<uint32_t> n_strata, gbase, bp;
    std::vector<uint64_t> weight;
    uint64_t W = 0;
    hipStream_t st = nullptr;
    int device = 0;
    dp::Plan p{};
    char* arena = nullptr;
    size_t arena_bytes = 0;
    bool noalloc = false;  // arena and staging are the device's static scratch and host buffer
    uint32_t* nstart = nullptr;
    uint32_t* hash_first = nullptr;  // tile -> first document table of the hash
    uint32_t* scan_base = nullptr;   // the scans' workspace (zeroed once at init)
    uint64_t scan_words = 0;
    uint32_t scan_epoch = 0;         // the last scan epoch (host)
    uint8_t* dig_buf = nullptr;
    size_t dig_cap = 0;
    // pinned host staging for every host<->device copy (asynchronous copies,
    // no pageable bounce); a bump allocator reset after each synchronization
    uint8_t* pin = nullptr;
    size_t pin_bytes = 0, pin_off = 0;
    // device mailbox mirroring the staging byte for byte: a batch of uploads
    // (downloads) is one copy of the staged span and one kernel that moves each
    // array to (from) its place
    uint8_t* mbox = nullptr;
    size_t mbox_bytes = 0;
    struct Moved {
        const uint8_t* src;
        uint8_t* dst;
        size_t off, bytes;  // staging offset and size
    };
    std::vector<Moved> upq, downq;
    std::vector<uint64_t> src_win_start, stats, checks, src_piece_start;
    std::vector<uint32_t> n_upd;
    int64_t cycle = -1;
    bool ready = false;  // a cycle is current: its device tables are valid for pack_batch
    uint32_t U = 0;
    std::vector<uint64_t> cyc_start, cyc_next, taken;
    // batch-size ramp: pieces, each piece's apportionment [K][S], the tokens
    // trained before the current cycle and after it, the cycle's per-update
    // batches and this rank's output prefix
    std::vector<uint64_t> ramp_from, ramp_tokens;
    std::vector<uint32_t> ramp_n_h;
    uint32_t* ramp_n = nullptr;        // device [K][S]
    dp::RampSpan* spans = nullptr;     // device [K+1]
    uint64_t tokens_start = 0, tokens_next = 0;
    std::vector<uint32_t> upd_B;
    std::vector<uint64_t> upd_out0;
    // lanes: the plan runs over S_real·lanes streams; the mixture over the real sources
    uint32_t lanes = 1, S_real = 0;
    std::vector<uint64_t> weight_real;
    std::vector<uint64_t> start_tokens;  // [S] first token of each stream, empty: from the start
    uint64_t* start_dev = nullptr;       // device copy
    uint64_t* next_win = nullptr;        // device [S]: first window of each stream's next cycle (~0: none)
    uint64_t* stream_next = nullptr;     // device [S]: its first token
    uint16_t* lane_source = nullptr;   // device [n_docs]: stream of each document
    uint32_t* n_real = nullptr;        // device [S_real]: one lane's apportionment
    uint32_t* nstart_real = nullptr;   // device [S_real+1]
    uint32_t* lane_src = nullptr;      // device [B/lanes]: one lane's slot table
    uint32_t* lane_k = nullptr;
    uint32_t* cum_Ar = nullptr;        // device [(U_cap+1)·S_real]: the per-lane schedule
    uint32_t* ramp_n_real = nullptr;   // device [K][S_real]
    std::string err;
};

namespace {

struct Carver {
    char* base;
    size_t off = 0;
    template <typename T>
    T* take(uint64_t count) {
        off = (off + ALIGN - 1) / ALIGN * ALIGN;
        T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
        off += sizeof(T) * (count ? count : 1);
        return p;
    }
};

size_t pin_bytes_for(uint32_t S, uint64_t K, uint64_t n_seg);

// smallest batch of an update: B, or the ramp's smallest piece
uint32_t ramp_bmin(const pack_ctx& c) {
    uint64_t b = c.p.B;
    for (uint64_t t : c.ramp_tokens) b = std::min<uint64_t>(b, t / c.p.T);
    return (uint32_t)b;
}

// Lay out (or size, when base == nullptr) every device array of the plan.
size_t carve(pack_ctx& c, char* base) {
    dp::Plan& p = c.p;
    const uint64_t D = p.n_docs, S = p.S, G = p.G, B = p.B, P = p.cap_pieces;
    Carver k{base};
    p.gbase = k.take<uint32_t>(S * p.n_seg + 1);
    p.n_strata = k.take<uint32_t>(S);
    p.weight = k.take<uint64_t>(c.S_real);  // the recipe's weights (read by the mixture over the real sources)
    p.bp = k.take<uint32_t>(S);
    // with the recipe (one staged copy at init): stream starts, zeroed statistics
    // and error flags, the pad row
    c.start_dev = k.take<uint64_t>(S);
    p.stats = k.take<uint64_t>(4 * S);
    p.err = k.take<uint32_t>(1);
    p.err_batch = k.take<uint32_t>(1);
    p.pad16 = k.take<uint32_t>(16);
    p.group = k.take<uint32_t>(D);
    p.hash = k.take<uint64_t>(D);
    c.hash_first = k.take<uint32_t>(dp::hash_tile_count(p.n_tokens) + 2);
    p.keep = k.take<uint8_t>(D);
    p.kept_pos = k.take<uint32_t>(D + 1);
    p.key[0] = k.take<uint64_t>(D);
    p.key[1] = k.take<uint64_t>(D);
    p.val[0] = k.take<uint32_t>(D);
    p.val[1] = k.take<uint32_t>(D);
    const uint64_t WR = p.read_random ? P : 0;  // cycle windows ≤ windows ≤ pieces
    {  // scans: kept flags (D), the sorts' bucket counts, lengths and pieces (≤ D)
        const uint64_t n_max = std::max<uint64_t>(D + 1, (D > WR ? D : WR) / 2 + (G > S ? G : S) + 1);
        c.scan_words = dp::scan_ws_bytes(n_max) / 4;
        c.scan_base = k.take<uint32_t>(c.scan_words);
        p.scan = dp::scan_ws_at(c.scan_base, n_max, p.err, &c.scan_epoch);
    }
    // right after the scan's words: build_plan zeroes both (and the padding
    // between) with one fill, the sort's counts for the compaction to count into
    p.hist = k.take<uint32_t>(dp::sort_hist_words(D > WR ? D : WR, G > S ? G : S));
    p.group_start = k.take<uint32_t>(G + 1);
    p.gpre = k.take<uint64_t>(D + 1);
    p.order = k.take<uint32_t>(D);
    p.src_doc_start = k.take<uint64_t>(S + 1);
    p.piece_start = k.take<uint32_t>(D + 1);
    p.opre = k.take<uint64_t>(D + 1);
    p.pc_doc = k.take<uint32_t>(P);
    p.pc_off = k.take<uint32_t>(P);
    p.pc_len = k.take<uint32_t>(P);
    p.pc_woff = k.take<uint32_t>(P);
    p.pc_emit = k.take<uint4>(P);
    p.pc_pre = k.take<uint64_t>(P + 1);
    p.src_piece_start = k.take<uint64_t>(S + 1);
    p.jump = k.take<uint32_t>((uint64_t)bitlen(P) * P);
    p.src_win_start = k.take<uint64_t>(S + 1);
    p.win_first = k.take<uint32_t>(P + 1);
    p.win_real = k.take<uint32_t>(P);
    p.win_learn = k.take<uint32_t>(P);
    p.n_upd = k.take<uint32_t>(S);
    p.slot_src = k.take<uint32_t>(B);
    p.slot_k = k.take<uint32_t>(B);
    p.cyc_start = k.take<uint64_t>(S);
    p.checks = k.take<uint64_t>(2);
    p.cyc_sums = k.take<uint64_t>(2);
    p.perm_start = k.take<uint64_t>(S + 1);
    p.perm = k.take<uint32_t>(WR);
    p.wkey[0] = k.take<uint64_t>(WR);
    p.wkey[1] = k.take<uint64_t>(WR);
    p.wval[0] = k.take<uint32_t>(WR);
    p.wval[1] = k.take<uint32_t>(WR);
    p.wgroup = k.take<uint32_t>(WR);
    // per-update tables: a cycle has at most P/Bmin updates (each takes ≥ Bmin of ≤ P windows)
    const uint64_t CU = p.tabled ? P / ramp_bmin(c) : 0;
    const uint64_t K = c.ramp_from.size();
    p.cum_A = k.take<uint32_t>(p.tabled ? (CU + 1) * S : 0);
    p.cum_rem = k.take<uint64_t>(p.tabled ? S : 0);
    p.cum_out = k.take<uint64_t>(p.tabled ? S + 1 : 0);
    p.cslot_src = k.take<uint32_t>(p.tabled ? P : 0);
    p.cslot_i = k.take<uint32_t>(p.tabled ? P : 0);
    p.upd_B = k.take<uint32_t>(p.ramp ? CU + 1 : 0);
    p.upd_slot0 = k.take<uint64_t>(p.ramp ? CU + 1 : 0);
    p.upd_out0 = k.take<uint64_t>(p.ramp ? CU + 1 : 0);
    c.ramp_n = k.take<uint32_t>(K * S);
    c.spans = k.take<dp::RampSpan>(K + 1);
    const bool lanes = c.lanes > 1;
    c.lane_source = k.take<uint16_t>(lanes ? D : 0);
    c.n_real = k.take<uint32_t>(c.S_real);
    c.nstart_real = k.take<uint32_t>(c.S_real + 1);
    c.lane_src = k.take<uint32_t>(B / c.lanes);
    c.lane_k = k.take<uint32_t>(B / c.lanes);
    c.cum_Ar = k.take<uint32_t>(lanes && p.cumulative ? (CU + 1) * c.S_real : 0);
    c.ramp_n_real = k.take<uint32_t>(K * c.S_real);
    c.next_win = k.take<uint64_t>(S);
    c.stream_next = k.take<uint64_t>(S);
    c.nstart = k.take<uint32_t>(S + 1);
    c.dig_cap = 128 + 72 * S + 16 * K + 28;  // records 60·S, header ≤ 100 + 16·K, leaves 32·⌈S/8⌉
    c.dig_buf = k.take<uint8_t>(c.dig_cap + 32);
    c.mbox_bytes = pin_bytes_for((uint32_t)S, K, p.n_seg);
    c.mbox = k.take<uint8_t>(c.mbox_bytes);
    // chunked window digests: 16 MiB of chunk digests, or those of a call's most windows (P ≥ a cycle's)
    p.chunk_cd_words = p.digest_chunked ? std::min<uint64_t>(4ull << 20, 8 * dp::digest_chunks(p.T) * std::max(P, B))
                                        : 0;
    p.chunk_cd = k.take<uint32_t>(p.chunk_cd_words);
    return k.off + ALIGN;
}

template <typename T>
void d2h(T* dst, const T* src, uint64_t count, hipStream_t st) {
    if (count) DP_HIP(hipMemcpyAsync(dst, src, sizeof(T) * count, hipMemcpyDeviceToHost, st));
}
template <typename T>
void h2d(T* dst, const T* src, uint64_t count, hipStream_t st) {
    if (count) DP_HIP(hipMemcpyAsync(dst, src, sizeof(T) * count, hipMemcpyHostToDevice, st));
}

// pinned staging: bytes for the largest set of copies between two synchronizations
// largest uses: pack_cycle's copies, each 64-byte aligned: cycle starts,
// read-order starts, the cumulative schedule's remaining windows and totals,
// next windows and next tokens (8·S bytes each, about 48·S in all), the ramp's
// spans (40 bytes per piece), sums, error flag, the plan digest's message (60·S
// bytes of stream records, then a header of at most 100 + 16·K bytes) and the
// digest; pack_init's first block (recipe with the arrival bases gbase,
// 4·(S·n_seg + 1) bytes, starts, statistics, pad row: ≤ 56·S + 4·S·n_seg bytes
// plus alignment)
size_t pin_bytes_for(uint32_t S, uint64_t K, uint64_t n_seg) {
    return 192ull * S + 112ull * K + 4ull * S * n_seg + 8192;
}

template <typename T>
T* pin_take(pack_ctx& c, uint64_t count) {
    c.pin_off = (c.pin_off + 63) / 64 * 64;
    T* p = reinterpret_cast<T*>(c.pin + c.pin_off);
    c.pin_off += sizeof(T) * (count ? count : 1);
    if (c.pin_off > c.pin_bytes) throw dp::HipError{hipErrorOutOfMemory, "internal: pinned staging exhausted"};
    return p;
}

// host array -> pinned staging -> device (asynchronous)
template <typename T>
void h2d_staged(pack_ctx& c, T* dst, const T* src, uint64_t count) {
    if (!count) return;
    T* h = pin_take<T>(c, count);
    std::memcpy(h, src, sizeof(T) * count);
    h2d(dst, h, count, c.st);
}

// device -> pinned staging (asynchronous); read the returned pointer after a synchronization
template <typename T>
T* d2h_staged(pack_ctx& c, const T* src, uint64_t count) {
    T* h = pin_take<T>(c, count);
    d2h(h, src, count, c.st);
    return h;
}

void flush_moved(pack_ctx& c, std::vector<pack_ctx::Moved>& q, bool upload) {
    if (q.empty()) return;
    size_t lo = ~size_t(0), hi = 0;
    dp::XferList l{};
    l.n = (uint32_t)q.size();
    for (uint32_t i = 0; i < l.n; ++i) {
        lo = std::min(lo, q[i].off);
        hi = std::max(hi, q[i].off + q[i].bytes);
        l.x[i] = dp::Xfer{q[i].src, q[i].dst, q[i].bytes};
    }
    q.clear();
    if (hi > c.mbox_bytes) throw dp::HipError{hipErrorOutOfMemory, "internal: transfer mailbox exhausted"};
    if (upload) {
        h2d(c.mbox + lo, c.pin + lo, hi - lo, c.st);
        dp::launch_xfer(l, c.st);
    } else {
        dp::launch_xfer(l, c.st);
        d2h(c.pin + lo, c.mbox + lo, hi - lo, c.st);
    }
}

// host array -> staging, queued; sent by up_flush (call it before the kernels that read dst)
template <typename T>
void up(pack_ctx& c, T* dst, const T* src, uint64_t count) {
    if (!count) return;
    T* h = pin_take<T>(c, count);
    std::memcpy(h, src, sizeof(T) * count);
    const size_t off = static_cast<size_t>(reinterpret_cast<uint8_t*>(h) - c.pin);
    c.upq.push_back({c.mbox + off, reinterpret_cast<uint8_t*>(dst), off, sizeof(T) * count});
    if (c.upq.size() == dp::XFER_MAX) flush_moved(c, c.upq, true);
}
void up_flush(pack_ctx& c) { flush_moved(c, c.upq, true); }

// device range -> staging, queued; read the returned pointer after sync_staged
template <typename T>
const T* down(pack_ctx& c, const T* src, uint64_t count) {
    T* h = pin_take<T>(c, count);
    if (!count) return h;
    const size_t off = static_cast<size_t>(reinterpret_cast<uint8_t*>(h) - c.pin);
    c.downq.push_back({reinterpret_cast<const uint8_t*>(src), c.mbox + off, off, sizeof(T) * count});
    if (c.downq.size() == dp::XFER_MAX) flush_moved(c, c.downq, false);
    return h;
}

void reset_staging(pack_ctx& c) {
    c.pin_off = 0;
    c.upq.clear();
    c.downq.clear();
}

// the queued downloads, then a synchronization; the staging is free again afterwards
void sync_staged(pack_ctx& c) {
    if (!c.upq.empty()) throw dp::HipError{hipErrorInvalidValue, "internal: uploads staged but not sent"};
    flush_moved(c, c.downq, false);
    DP_HIP(hipStreamSynchronize(c.st));
    reset_staging(c);
}

void check_config(const pack_config* cfg) {
    auto bad = [](const char* m) { throw InvalError{m}; };
    if (cfg->flags &
        ~(PACK_FLAG_TIMING | PACK_FLAG_TIMING_BATCH | PACK_FLAG_WRAP | PACK_FLAG_HELDOUT | PACK_FLAG_READ_RANDOM |
          PACK_FLAG_CUMULATIVE | PACK_FLAG_DIGEST_CHUNKED))
        bad("unknown flags");
    if (cfg->n_docs < 1 || cfg->n_docs >= (1ull << 31)) bad("n_docs must be in [1, 2^31)");
    if (!cfg->doc_offsets || !cfg->doc_source) bad("doc_offsets and doc_source are required");
    if (cfg->n_tokens && !cfg->tokens) bad("tokens is NULL with n_tokens > 0");
    if (cfg->n_tokens >= (1ull << dp::SCAN_VALUE_BITS)) bad("n_tokens must be below 2^40");
    if (cfg->n_sources < 1 || cfg->n_sources > 4096) bad("n_sources must be in [1, 4096]");
    if (!cfg->share_weight || !cfg->holdout_bp) bad("share_weight and holdout_bp are required");
    const uint32_t T = cfg->window_tokens, B = cfg->global_batch;
    if (T < 1 || T > (1u << 20)) bad("window_tokens must be in [1, 2^20]");
    if (B < 1 || B > (1u << 20)) bad("global_batch must be in [1, 2^20]");
    if (cfg->world < 1 || cfg->rank >= cfg->world) bad("need world >= 1 and rank < world");
    if (B % cfg->world) bad("world must divide global_batch");
    uint64_t G = 0;
    for (uint32_t s = 0; s < cfg->n_sources; ++s) {
        const uint32_t k = cfg->n_strata ? cfg->n_strata[s] : 1u;
        if (k < 1) bad("every source needs at least one stratum");
        G += k;
        if (cfg->holdout_bp[s] > 10000) bad("holdout_bp must be <= 10000");
    }
    const uint64_t NSEG = cfg->doc_segment && cfg->n_segments > 1 ? cfg->n_segments : 1;
    if (cfg->n_segments > 65536) bad("at most 65536 arrivals");
    if (G * NSEG > 65536) bad("at most 65536 (source, arrival, stratum) groups");
    unsigned __int128 W = 0;
    for (uint32_t s = 0; s < cfg->n_sources; ++s) W += cfg->share_weight[s];
    if (W == 0 || (W >> 64) != 0) bad("share weights must sum to [1, 2^64)");
    uint32_t Bmin = B;
    if (cfg->n_ramp) {
        if (cfg->n_ramp > 4096) bad("at most 4096 ramp pieces");
        if (!cfg->ramp_from || !cfg->ramp_tokens) bad("ramp_from and ramp_tokens are required with n_ramp > 0");
        uint64_t Bmax = 0;
        for (uint32_t k = 0; k < cfg->n_ramp; ++k) {
            const uint64_t tk = cfg->ramp_tokens[k];
            if (tk == 0 || tk % T) bad("every ramp piece's tokens per update must be a positive multiple of T");
            const uint64_t Bk = tk / T;
            if (Bk > (1u << 20)) bad("a ramp piece's batch must be at most 2^20 windows");
            if (Bk % cfg->world) bad("world must divide every ramp piece's batch");
            if (k == 0 ? cfg->ramp_from[0] != 0 : cfg->ramp_from[k] <= cfg->ramp_from[k - 1])
                bad("ramp pieces must start at 0 tokens and rise");
            if (Bk > Bmax) Bmax = Bk;
            if (Bk < Bmin) Bmin = (uint32_t)Bk;
        }
        if (Bmax != B) bad("with a ramp, global_batch must be the largest piece's batch");
    }
    if (cfg->flags & PACK_FLAG_CUMULATIVE) {
        if (cfg->n_sources > 1024) bad("the cumulative mixture takes at most 1024 sources");
        for (uint32_t s = 0; s < cfg->n_sources; ++s)  // every due update then lies within 2^62 updates
            if (cfg->share_weight[s] && ((unsigned __int128)cfg->share_weight[s] << 62) <= W)
                bad("the cumulative mixture needs every nonzero share to be at least 2^-62 of the weights");
    }
    const uint32_t L = cfg->n_lanes > 1 ? cfg->n_lanes : 1;
    if (L > 1) {
        if (B % L) bad("lanes must divide global_batch");
        for (uint32_t k = 0; k < cfg->n_ramp; ++k)
            if ((cfg->ramp_tokens[k] / T) % L) bad("lanes must divide every ramp piece's batch");
        if (L % cfg->world) bad("world must divide the lanes (each rank takes whole lanes)");
        if ((uint64_t)cfg->n_sources * L > 4096) bad("n_sources x lanes must be at most 4096");
        if (G * L * NSEG > 65536) bad("(source, arrival, stratum) groups x lanes must be at most 65536");
    }
    if ((cfg->flags & PACK_FLAG_CUMULATIVE) || cfg->n_ramp) {
        const uint64_t cap = cfg->n_docs + cfg->n_tokens / T;  // windows ≤ pieces ≤ cap
        if ((cap / Bmin + 1) * cfg->n_sources * L > (1ull << 28))
            bad("the per-update table (updates x streams) exceeds 2^28 entries");
    }
}

int fail_hip(pack_ctx* c, const dp::HipError& e) {
    const std::string m = std::string(e.what) + ": " + hipGetErrorString(e.code);
    if (c) c->err = m;
    else g_init_error = m;
    return PACK_E_HIP;
}

void release(pack_ctx* c) {
    if (!c) return;
    if (c->arena || c->pin) (void)hipStreamSynchronize(c->st);
    if (c->noalloc) {  // static memory: hand the device's slot back, never to the arena cache
        std::lock_guard<std::mutex> lk(g_noalloc_mu);
        g_noalloc[c->device].in_use = false;
    } else {
        if (c->arena) arena_give(c->device, c->arena, c->arena_bytes);
        if (c->pin) arena_give(c->device, c->pin, c->pin_bytes, true);
    }
    c->timer.destroy();
    delete c;
}

void build_plan(pack_ctx& c) {
    dp::Plan& p = c.p;
    hipStream_t st = c.st;
    // the recipe, stream starts, zeroed statistics and error flag and the pad
    // row lie together at the start of the workspace: laid out in the pinned
    // staging area as on the device and sent with one copy
    reset_staging(c);
    {
        uint8_t* const dbase = reinterpret_cast<uint8_t*>(p.gbase);
        const size_t span = static_cast<size_t>(reinterpret_cast<uint8_t*>(p.pad16 + 16) - dbase);
        uint8_t* const h = pin_take<uint8_t>(c, span);
        std::memset(h, 0, span);
        auto place = [&](const void* dev, const void* src, size_t bytes) {
            if (bytes) std::memcpy(h + (static_cast<const uint8_t*>(dev) - dbase), src, bytes);
        };
        place(p.gbase, c.gbase.data(), 4ull * ((uint64_t)p.S * p.n_seg + 1));
        place(p.n_strata, c.n_strata.data(), 4ull * p.S);
        place(p.weight, c.weight_real.data(), 8ull * c.S_real);
        place(p.bp, c.bp.data(), 4ull * p.S);
        if (!c.start_tokens.empty()) {
            place(c.start_dev, c.start_tokens.data(), 8ull * p.S);
            p.start_tok = c.start_dev;
        }
        uint32_t* const pad = reinterpret_cast<uint32_t*>(h + (reinterpret_cast<uint8_t*>(p.pad16) - dbase));
        for (int i = 0; i < 16; ++i) pad[i] = p.pad_token;
        h2d(dbase, h, span, st);
    }

    // validation first: no kernel reads the corpus through unchecked offsets
    c.timer.begin(PACK_PHASE_VALIDATE, st);
    // no tile ticket taken, no status published; the plan sort's group and
    // bucket counts zeroed (they lie right after the scan's words)
    dp::launch_zero_u32(c.scan_base, static_cast<uint64_t>(p.hist - c.scan_base) + dp::sort_count_words(p.n_docs, p.G),
                        st);
    c.scan_epoch = 0;
    if (c.lanes > 1) {  // documents to streams (source, lane); the validation then checks stream ids
        dp::launch_lane_source(c.cfg.doc_source, p.n_docs, c.S_real, c.lanes, c.lane_source, st);
        p.source = c.lane_source;
    }
    // the validation also zeroes the hash's per-document sums (gpre, free
    // until the merge) and writes its tile table
    dp::launch_validate(p, p.gpre, c.hash_first, st);
    c.timer.end(st);

    // A1 hash + hold-out, A2 compaction, A3 keys; after an invalid corpus the
    // hash kernels return at once (they read the error flag) and the error is
    // raised below, before any later kernel runs
    c.timer.begin(PACK_PHASE_HASH, st);
    dp::launch_hash(p, p.gpre, c.hash_first, st);
    c.timer.end(st);
    c.timer.begin(PACK_PHASE_KEYS, st);
    dp::launch_keep_scan(p, st);
    c.timer.end(st);
    const uint32_t* h_err = down(c, p.err, 1);
    const uint32_t* h_kept = down(c, p.kept_pos + p.n_docs, 1);
    sync_staged(c);
    uint32_t err = *h_err;
    if (err & dp::ERR_INTERNAL) throw InternalError{"internal: a scan's bounded wait gave up (library bug)"};
    if (err) {
        std::string m = "invalid corpus:";
        if (err & 1u) m += " offsets decrease;";
        if (err & 2u) m += " a document has 2^32 or more tokens;";
        if (err & 4u) m += " a source id >= n_sources;";
        if (err & 8u) m += " a stratum id >= n_strata of its source;";
        if (err & 16u) m += " doc_offsets[n_docs] > n_tokens;";
        if (err & 32u) m += " an arrival id >= n_segments;";
        throw InvalError{m};
    }
    p.n_kept = *h_kept;

    // A3 sort, A4 merge, A5 piece counts
    c.timer.begin(PACK_PHASE_SORT, st);
    dp::launch_sort(p, st);
    c.timer.end(st);
    c.timer.begin(PACK_PHASE_MERGE, st);
    dp::launch_merge(p, st);
    c.timer.end(st);
    c.timer.begin(PACK_PHASE_PIECES, st);
    dp::launch_piece_count(p, st);
    c.timer.end(st);
    // the piece and window counts stay on the device until the end: the
    // launches below are sized by their bound and the kernels read the counts
    p.n_pieces_dev = p.piece_start + p.n_kept;
    p.n_windows_dev = p.src_win_start + p.S;
    p.n_pieces = p.n_windows = p.cap_pieces;
    p.levels = bitlen(p.cap_pieces) ? bitlen(p.cap_pieces) : 1;

    // A5 pieces, next-fit by lifting, windows per source
    c.timer.begin(PACK_PHASE_PIECES, st);
    dp::launch_pieces(p, st);
    c.timer.end(st);
    c.timer.begin(PACK_PHASE_CUT, st);
    dp::launch_lifting(p, st);
    dp::launch_window_count(p, st);
    c.timer.end(st);

    // window table, A6 mixture, checks
    c.timer.begin(PACK_PHASE_WINDOWS, st);
    dp::launch_zero_u32(p.win_first, 1, st);  // an empty plan still has win_first[0] = 0
    dp::launch_windows(p, st);
    c.timer.end(st);
    c.timer.begin(PACK_PHASE_MIXTURE, st);
    {
        // one lane's mixture over the recipe's sources (B/L windows), then every lane the same
        dp::Plan pr = p;
        pr.S = c.S_real;
        pr.B = p.B / c.lanes;
        if (c.lanes > 1) {
            pr.n_upd = c.n_real;
            pr.slot_src = c.lane_src;
            pr.slot_k = c.lane_k;
            dp::launch_mixture_w(pr, c.W, c.nstart_real, st);
            dp::launch_lane_expand(p, c.n_real, c.lane_src, c.lane_k, st);
        } else {
            dp::launch_mixture_w(p, c.W, c.nstart, st);
        }
        for (size_t k = 0; k < c.ramp_tokens.size(); ++k)  // each ramp piece's lane batch apportioned the same way
            dp::launch_apportion(pr, c.W, (uint32_t)(c.ramp_tokens[k] / p.T / c.lanes), c.ramp_n_real + k * c.S_real,
                                 st);
    }
    dp::launch_checks(p, st);
    c.timer.end(st);
    // the plan's counts back to the host: one gather kernel and one copy
    const uint32_t* h_upd = down(c, p.n_upd, p.S);
    const uint64_t* h_stats = down(c, p.stats, 4ull * p.S);
    const uint64_t* h_checks = down(c, p.checks, 2);
    const uint64_t* h_sps = down(c, p.src_piece_start, p.S + 1);
    const uint32_t* h_pieces = down(c, p.piece_start + p.n_kept, 1);
    const uint64_t* h_sws = down(c, p.src_win_start, p.S + 1);
    h_err = down(c, p.err, 1);
    sync_staged(c);
    p.n_pieces_dev = nullptr;  // host counts from here on
    p.n_windows_dev = nullptr;
    p.n_pieces = *h_pieces;
    if (p.n_pieces > p.cap_pieces) throw InvalError{"internal: piece bound exceeded"};
    c.src_win_start.assign(h_sws, h_sws + p.S + 1);
    p.n_windows = c.src_win_start[p.S];
    c.n_upd.assign(h_upd, h_upd + p.S);
    c.stats.assign(h_stats, h_stats + 4ull * p.S);
    c.checks.assign(h_checks, h_checks + 2);
    c.src_piece_start.assign(h_sps, h_sps + p.S + 1);
    err = *h_err;
    if (err) throw InternalError{"internal plan consistency check failed (library bug)"};
    if (!c.ramp_tokens.empty()) {  // K·S counts: once, at init (may exceed the staging area)
        const uint64_t K = c.ramp_tokens.size();
        std::vector<uint32_t> nr(K * c.S_real);
        d2h(nr.data(), c.ramp_n_real, nr.size(), st);
        DP_HIP(hipStreamSynchronize(st));
        c.ramp_n_h.resize(K * p.S);  // every lane of a source the same count
        for (uint64_t k = 0; k < K; ++k)
            for (uint32_t v = 0; v < p.S; ++v) c.ramp_n_h[k * p.S + v] = nr[k * c.S_real + v / c.lanes];
        h2d(c.ramp_n, c.ramp_n_h.data(), c.ramp_n_h.size(), st);
        DP_HIP(hipStreamSynchronize(st));
    }
}

void put(std::vector<uint8_t>& b, uint64_t v, int bytes) {
    for (int i = 0; i < bytes; ++i) b.push_back((uint8_t)(v >> (8 * i)));
}

}  // namespace

namespace {

int init_context(const pack_config* cfg, pack_ctx** out, bool noalloc) {
    g_init_error.clear();
    if (!out) {
        g_init_error = "out is NULL";
        return PACK_E_INVAL;
    }
    *out = nullptr;
    if (!cfg) {
        g_init_error = "cfg is NULL";
        return PACK_E_INVAL;
    }
    if (cfg->abi_version != DPACK_ABI_VERSION) {
        g_init_error = "abi_version mismatch";
        return PACK_E_ABI;
    }
    if (noalloc && (cfg->flags & (PACK_FLAG_TIMING | PACK_FLAG_TIMING_BATCH))) {  // events are created per context
        g_init_error = "pack_init_noalloc does not take PACK_FLAG_TIMING or PACK_FLAG_TIMING_BATCH";
        return PACK_E_INVAL;
    }
    pack_ctx* c = nullptr;
    try {
        check_config(cfg);
        c = new (std::nothrow) pack_ctx;
        if (!c) {
            g_init_error = "host allocation failed";
            return PACK_E_NOMEM;
        }
        c->cfg = *cfg;
        c->cycle = (int64_t)cfg->first_cycle - 1;
        if (cfg->start_tokens)
            c->start_tokens.assign(cfg->start_tokens, cfg->start_tokens + (uint64_t)cfg->n_sources *
                                                                              (cfg->n_lanes > 1 ? cfg->n_lanes : 1));
        c->st = static_cast<hipStream_t>(cfg->stream);
        c->timer.on = (cfg->flags & (PACK_FLAG_TIMING | PACK_FLAG_TIMING_BATCH)) != 0;
        c->timer.phases = (cfg->flags & PACK_FLAG_TIMING) ? (1u << PACK_N_PHASES) - 1u
                                                           : (1u << PACK_PHASE_EMIT) | (1u << PACK_PHASE_LEARNED) |
                                                                 (1u << PACK_PHASE_DIGEST) |
                                                                 (1u << PACK_PHASE_FINGERPRINT);
        // with lanes, every per-source array is per stream s·L + l (the recipe's values per source)
        const uint32_t L = cfg->n_lanes > 1 ? cfg->n_lanes : 1, Sr = cfg->n_sources, S = Sr * L;
        c->lanes = L;
        c->S_real = Sr;
        c->weight_real.assign(cfg->share_weight, cfg->share_weight + Sr);
        const uint32_t NSEG = cfg->doc_segment && cfg->n_segments > 1 ? cfg->n_segments : 1;
        c->n_strata.resize(S);
        c->gbase.resize((uint64_t)S * NSEG + 1);
        c->bp.resize(S);
        c->weight.resize(S);
        uint32_t G = 0;
        for (uint32_t s = 0; s < S; ++s) {
            c->n_strata[s] = cfg->n_strata ? cfg->n_strata[s / L] : 1u;
            c->bp[s] = cfg->holdout_bp[s / L];
            c->weight[s] = cfg->share_weight[s / L];
        }
        for (uint32_t u = 0; u < S * NSEG; ++u) {  // groups (stream, arrival, stratum)
            c->gbase[u] = G;
            G += c->n_strata[u / NSEG];
        }
        for (uint32_t r = 0; r < Sr; ++r) c->W += c->weight_real[r];
        c->gbase[(uint64_t)S * NSEG] = G;

        dp::Plan& p = c->p;
        p.tokens = cfg->tokens;
        p.offsets = cfg->doc_offsets;
        p.source = cfg->doc_source;
        p.stratum = cfg->doc_stratum;
        p.prompt_len = cfg->doc_prompt_len;
        p.segment = NSEG > 1 ? cfg->doc_segment : nullptr;
        p.n_seg = NSEG;
        p.n_tokens = cfg->n_tokens;
        p.n_docs = cfg->n_docs;
        p.S = S;
        p.G = G;
        p.T = cfg->window_tokens;
        p.B = cfg->global_batch;
        p.seed = cfg->seed;
        p.pad_token = cfg->pad_token;
        p.wrap = (cfg->flags & PACK_FLAG_WRAP) ? 1u : 0u;
        p.heldout = (cfg->flags & PACK_FLAG_HELDOUT) ? 1u : 0u;
        p.read_random = (cfg->flags & PACK_FLAG_READ_RANDOM) ? 1u : 0u;
        p.cumulative = (cfg->flags & PACK_FLAG_CUMULATIVE) ? 1u : 0u;
        p.digest_chunked = (cfg->flags & PACK_FLAG_DIGEST_CHUNKED) ? 1u : 0u;
        p.ramp = cfg->n_ramp ? 1u : 0u;
        p.tabled = (p.cumulative || p.ramp) ? 1u : 0u;
        p.world = cfg->world;
        p.lanes = L;
        p.S_real = Sr;
        c->ramp_from.assign(cfg->ramp_from, cfg->ramp_from + cfg->n_ramp);
        c->ramp_tokens.assign(cfg->ramp_tokens, cfg->ramp_tokens + cfg->n_ramp);
        p.cap_pieces = cfg->n_docs + cfg->n_tokens / cfg->window_tokens;
        if (p.cap_pieces >= 0xFFFFFFFFull) throw InvalError{"too many pieces for 32-bit piece indices"};

        const size_t bytes = carve(*c, nullptr);
        const size_t pbytes = pin_bytes_for(S, cfg->n_ramp, c->p.n_seg);
        if (noalloc && (bytes > NOALLOC_DEVICE_BYTES || pbytes > NOALLOC_HOST_BYTES)) {
            // the static workspace's limits, before any device work
            g_init_error = "pack_init_noalloc: the plan needs " + std::to_string(bytes) +
                           " bytes of device workspace and " + std::to_string(pbytes) +
                           " bytes of staging; the static scratch holds " +
                           std::to_string(NOALLOC_DEVICE_BYTES) + " and " + std::to_string(NOALLOC_HOST_BYTES);
            delete c;
            return PACK_E_INVAL;
        }
        DP_HIP(hipGetDevice(&c->device));
        if (noalloc) {
            if (c->device < 0 || c->device >= NOALLOC_MAX_DEVICES) {
                g_init_error = "pack_init_noalloc: device index beyond the static slots";
                delete c;
                return PACK_E_INVAL;
            }
            std::lock_guard<std::mutex> lk(g_noalloc_mu);
            NoallocSlot& slot = g_noalloc[c->device];
            if (slot.in_use) {
                g_init_error = "pack_init_noalloc: a context made by it is still alive on this device";
                delete c;
                return PACK_E_STATE;
            }
            if (!slot.dev) {  // once per device, with that device current
                void* ptr = nullptr;
                const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
                if (e != hipSuccess || !ptr) {
                    (void)hipGetLastError();
                    g_init_error = std::string("pack_init_noalloc: hipGetSymbolAddress(scratch): ") +
                                   hipGetErrorString(e);
                    delete c;
                    return PACK_E_HIP;
                }
                slot.dev = ptr;
            }
            slot.in_use = true;
            c->noalloc = true;
            c->arena = static_cast<char*>(slot.dev);
            c->arena_bytes = NOALLOC_DEVICE_BYTES;
            c->pin = slot.host;
            c->pin_bytes = NOALLOC_HOST_BYTES;
            carve(*c, c->arena);
        } else {
            size_t got = 0;
            void* mem = arena_take(c->device, bytes, &got);
            if (!mem) {
                if (hipMalloc(&mem, bytes) != hipSuccess) {
                    (void)hipGetLastError();
                    g_init_error = "device workspace allocation failed (" + std::to_string(bytes) + " bytes)";
                    delete c;
                    return PACK_E_NOMEM;
                }
                got = bytes;
            }
            c->arena = static_cast<char*>(mem);
            c->arena_bytes = got;
            carve(*c, c->arena);
            void* pin = arena_take(c->device, pbytes, &got, true);
            if (!pin) {
                if (hipHostMalloc(&pin, pbytes, hipHostMallocDefault) != hipSuccess) {
                    (void)hipGetLastError();
                    g_init_error = "pinned host staging allocation failed";
                    release(c);
                    return PACK_E_NOMEM;
                }
                got = pbytes;
            }
            c->pin = static_cast<uint8_t*>(pin);
            c->pin_bytes = got;
        }
        build_plan(*c);
        c->cyc_start.assign(S, 0);
        c->cyc_next.assign(S, 0);
        c->taken.assign(S, 0);
        *out = c;
        return PACK_OK;
    } catch (const InvalError& e) {
        g_init_error = e.msg;
        release(c);
        return PACK_E_INVAL;
    } catch (const InternalError& e) {
        g_init_error = e.msg;
        release(c);
        return PACK_E_INTERNAL;
    } catch (const dp::HipError& e) {
        fail_hip(nullptr, e);
        release(c);
        return PACK_E_HIP;
    } catch (const std::bad_alloc&) {
        g_init_error = "host allocation failed";
        release(c);
        return PACK_E_NOMEM;
    }
}

}  // namespace

extern "C" {

const char* pack_strerror(int code) {
    switch (code) {
        case PACK_OK: return "ok";
        case PACK_E_ABI: return "ABI version mismatch";
        case PACK_E_INVAL: return "invalid argument or corpus";
        case PACK_E_NOMEM: return "out of memory";
        case PACK_E_HIP: return "HIP runtime error";
        case PACK_E_EXHAUSTED: return "a source cannot supply the cycle (data exhausted)";
        case PACK_E_STATE: return "call out of order";
        case PACK_E_RANGE: return "step range outside the current cycle";
        case PACK_E_INTERNAL: return "internal failure inside a kernel (library bug); results not valid";
        default: return "unknown error";
    }
}

const char* pack_last_error(const pack_ctx* ctx) {
    return ctx ? ctx->err.c_str() : g_init_error.c_str();
}

int pack_init(const pack_config* cfg, pack_ctx** out) { return init_context(cfg, out, false); }

int pack_init_noalloc(const pack_config* cfg, pack_ctx** out) { return init_context(cfg, out, true); }

int pack_cycle(pack_ctx* c, uint32_t cycle, pack_cycle_info* info) {
    if (!c) return PACK_E_INVAL;
    c->err.clear();
    const uint32_t S = c->p.S;
    if ((int64_t)cycle != c->cycle + 1) {
        c->err = "cycles must be planned in order first_cycle, first_cycle + 1, ...";
        return PACK_E_STATE;
    }
    // From here the cycle's device tables are rewritten: until this call
    // succeeds no cycle is current.  Host state is committed only after the
    // final synchronization, so on any error the same cycle can be planned again.
    c->ready = false;
    try {
        std::vector<uint64_t> start(S), rem(S), taken(S);
        for (uint32_t s = 0; s < S; ++s) {
            start[s] = cycle == c->cfg.first_cycle ? 0 : c->cyc_next[s];
            rem[s] = c->src_win_start[s + 1] - c->src_win_start[s] - start[s];
        }
        dp::Plan& p = c->p;
        uint64_t U = c->cfg.updates_per_cycle;
        const uint64_t* h_sums = nullptr;
        reset_staging(*c);
        // tokens trained before the cycle
        const uint64_t t0 = cycle == c->cfg.first_cycle ? c->cfg.tokens_start : c->tokens_next;
        std::vector<uint32_t> upd_B;
        std::vector<uint64_t> upd_out0;
        // cycle kernels flag internal failures in err: zeroed here when kernels run before the
        // uploads below (ramp, cumulative schedule), else with the uploads
        if (p.tabled) dp::launch_zero_u32(p.err, 1, c->st);
        if (p.tabled) {
            // per-update counts: the cumulative schedule and/or a batch-size ramp
            uint64_t total = 0;
            for (uint32_t s = 0; s < S; ++s) total += rem[s];
            const uint32_t Bmin = ramp_bmin(*c);
            const uint64_t most = total / Bmin;  // every update takes at least Bmin windows
            if (most == 0 || U > most) {
                c->err = "a source cannot supply the cycle's windows";
                return PACK_E_EXHAUSTED;
            }
            const uint64_t cap = U ? U : most;
            if (cap > p.cap_pieces / Bmin) throw InvalError{"internal: per-update table bound exceeded"};
            std::vector<dp::RampSpan> spans;
            if (p.ramp) {  // the ramp's pieces from the tokens trained so far, the last without end
                const uint64_t K = c->ramp_from.size();
                uint64_t u = 0, t = t0, slot = 0, out = 0;
                for (;;) {
                    uint32_t k = (uint32_t)(std::upper_bound(c->ramp_from.begin(), c->ramp_from.end(), t) -
                                            c->ramp_from.begin()) - 1;
                    const uint64_t tk = c->ramp_tokens[k], Bk = tk / p.T;
                    spans.push_back(dp::RampSpan{u, slot, out, (uint32_t)Bk, k});
                    if (k + 1 == K) break;
                    const uint64_t n = (c->ramp_from[k + 1] - t + tk - 1) / tk;  // updates of piece k
                    u += n;
                    t += n * tk;
                    slot += n * Bk;
                    out += n * (Bk / c->cfg.world);
                }
                h2d_staged(*c, c->spans, spans.data(), spans.size());
                dp::launch_ramp_fill(p, c->spans, (uint32_t)spans.size(), cap, c->st);
                p.spans = c->spans;
                p.n_spans = (uint32_t)spans.size();
            }
            if (p.cumulative) {  // the cycle's schedule from its cumulative quotas, on the device
                // one schedule over the recipe's sources with B/L seats per update, which every lane
                // follows: it must fit the lane of each source with the fewest windows left
                const uint32_t L = c->lanes, Sr = c->S_real;
                std::vector<uint64_t> rr(Sr, ~0ull);
                for (uint32_t v = 0; v < S; ++v) rr[v / L] = std::min(rr[v / L], rem[v]);
                dp::Plan pc = p;
                pc.S = Sr;
                if (L > 1) pc.cum_A = c->cum_Ar;
                // integral quotas (every update's seats times every weight a multiple of W):
                // the schedule has a closed form
                bool integral = true;
                for (uint32_t r = 0; r < Sr && integral; ++r) {
                    const unsigned __int128 w = c->weight_real[r];
                    if (p.ramp) {
                        for (const dp::RampSpan& sp : spans) integral = integral && (sp.B / L) * w % c->W == 0;
                    } else {
                        integral = (p.B / L) * w % c->W == 0;
                    }
                }
                c->timer.begin(PACK_PHASE_CYCLE, c->st);
                h2d_staged(*c, p.cum_rem, rr.data(), Sr);
                dp::launch_cumulative(pc, c->W, cap, integral, c->st);
                c->timer.end(c->st);
                const uint64_t* h_out = d2h_staged(*c, p.cum_out, Sr + 1);
                const uint32_t* h_err = d2h_staged(*c, p.err, 1);
                sync_staged(*c);
                if (*h_err & dp::ERR_INTERNAL) throw InternalError{"internal: cumulative schedule (library bug)"};
                const uint64_t got = h_out[Sr];
                for (uint32_t v = 0; v < S; ++v) taken[v] = h_out[v / L];
                reset_staging(*c);
                if (got == 0 || (U && got < U)) {
                    c->err = "a source cannot supply the cycle's windows";
                    return PACK_E_EXHAUSTED;
                }
                U = got;
                if (L > 1) dp::launch_cum_expand(p, c->cum_Ar, U, c->st);
            } else {  // the fixed apportionment of each update's batch: per source, the updates it supports
                uint64_t fit = cap;
                for (uint32_t s = 0; s < S; ++s) {
                    uint64_t a = 0;
                    for (size_t x = 0; x < spans.size() && spans[x].first < cap; ++x) {
                        const uint64_t end = x + 1 < spans.size() ? std::min<uint64_t>(spans[x + 1].first, cap) : cap;
                        const uint64_t n = c->ramp_n_h[(uint64_t)spans[x].k * S + s], len = end - spans[x].first;
                        if (n && a + len * n > rem[s]) {
                            fit = std::min<uint64_t>(fit, spans[x].first + (rem[s] - a) / n);
                            break;
                        }
                        a += len * n;
                    }
                }
                if (fit == 0 || (U && fit < U)) {
                    c->err = "a source cannot supply the cycle's windows";
                    return PACK_E_EXHAUSTED;
                }
                U = U ? U : fit;
                for (uint32_t s = 0; s < S; ++s) {
                    uint64_t a = 0;
                    for (size_t x = 0; x < spans.size() && spans[x].first < U; ++x) {
                        const uint64_t end = x + 1 < spans.size() ? std::min<uint64_t>(spans[x + 1].first, U) : U;
                        a += (end - spans[x].first) * c->ramp_n_h[(uint64_t)spans[x].k * S + s];
                    }
                    taken[s] = a;
                }
                dp::launch_ramp_fixed_A(p, c->spans, (uint32_t)spans.size(), c->ramp_n, U, c->st);
            }
            if (U > 0xFFFFFFFFull) throw InvalError{"internal: updates per cycle"};
            if (p.ramp) {  // host copies of the cycle's batches and this rank's output prefix
                upd_B.resize(U);
                upd_out0.assign(U + 1, 0);
                for (size_t x = 0; x < spans.size(); ++x) {
                    const uint64_t end = x + 1 < spans.size() ? std::min<uint64_t>(spans[x + 1].first, U) : U;
                    for (uint64_t u = spans[x].first; u < end; ++u) {
                        upd_B[u] = spans[x].B;
                        upd_out0[u + 1] = upd_out0[u] + spans[x].B / c->cfg.world;
                    }
                }
            }
        } else {
            if (U == 0) {
                U = ~0ull;
                for (uint32_t s = 0; s < S; ++s) {
                    if (c->n_upd[s] == 0) continue;
                    const uint64_t u = rem[s] / c->n_upd[s];
                    if (u < U) U = u;
                }
            }
            bool ok = U > 0 && U <= 0xFFFFFFFFull;
            for (uint32_t s = 0; ok && s < S; ++s)
                if ((unsigned __int128)U * c->n_upd[s] > (unsigned __int128)rem[s]) ok = false;
            if (!ok) {
                c->err = "a source cannot supply the cycle's windows";
                return PACK_E_EXHAUSTED;
            }
            for (uint32_t s = 0; s < S; ++s) taken[s] = U * c->n_upd[s];
        }
        uint64_t slots = 0;  // windows of the cycle, all ranks
        if (p.ramp)
            for (uint32_t b : upd_B) slots += b;
        else
            slots = U * p.B;
        const uint32_t U32 = (uint32_t)U;
        std::vector<uint64_t> next(S);
        for (uint32_t s = 0; s < S; ++s) next[s] = start[s] + taken[s];
        // every upload of the cycle is computed on the host first: the stream
        // starts, the read order's source starts, each stream's next window
        // and the plan digest's message go to the device together
        std::vector<uint64_t> ps;
        if (p.read_random) {  // each source's cycle windows in their random read order
            ps.assign(S + 1, 0);
            for (uint32_t s = 0; s < S; ++s) ps[s + 1] = ps[s] + taken[s];
        }
        std::vector<uint64_t> nw(S);  // each stream's first window of the next cycle
        for (uint32_t s = 0; s < S; ++s) {
            const uint64_t M = c->src_win_start[s + 1] - c->src_win_start[s];
            nw[s] = next[s] < M ? c->src_win_start[s] + next[s] : ~0ull;
        }

        // plan digest: SHA-256 of a little-endian header (mode, the recipe's
        // scalars, the cycle, its updates, two order-free sums over the plan)
        // followed by the digests of the streams' 60-byte records, 8 streams
        // to a leaf (one wavefront each), so the serial chain stays short: a
        // leaf is 8 blocks, and the top hash grows by one block per 2 leaves.
        // The records, then the header, go to the device with the cycle's
        // other uploads; the leaf digests are written after the header there.
        constexpr uint32_t REC = 60, LEAF = 8;
        std::vector<uint8_t> msg;
        for (uint32_t s = 0; s < S; ++s) {
            put(msg, c->weight[s], 8);
            put(msg, c->bp[s], 4);
            put(msg, c->n_strata[s], 4);
            put(msg, c->n_upd[s], 4);
            put(msg, c->src_win_start[s + 1] - c->src_win_start[s], 8);
            put(msg, c->stats[0 * S + s], 8);
            put(msg, c->stats[1 * S + s], 8);
            put(msg, start[s], 8);
            put(msg, c->start_tokens.empty() ? 0 : c->start_tokens[s], 8);
        }
        const size_t rec_bytes = msg.size();  // REC · S
        // the packing mode (D next-fit, W wrap) and the stream (1 training, V held-out) are part of the plan
        const char magic[8] = {'D', 'P', 'A', 'C', 'K', 'P', p.wrap ? 'W' : 'D', p.heldout ? 'V' : '1'};
        msg.insert(msg.end(), magic, magic + 8);
        if (p.read_random) put(msg, 0x444E4152u, 4);  // "RAND": windows read in a random order
        if (p.cumulative) put(msg, 0x554D5543u, 4);   // "CUMU": per-update counts from cumulative quotas
        if (p.ramp) {                                  // "RAMP": the pieces and the cycle's first token
            put(msg, 0x504D4152u, 4);
            put(msg, c->ramp_from.size(), 4);
            for (size_t k = 0; k < c->ramp_from.size(); ++k) {
                put(msg, c->ramp_from[k], 8);
                put(msg, c->ramp_tokens[k], 8);
            }
            put(msg, t0, 8);
        }
        if (c->lanes > 1) {                            // "LANE" and the lane count
            put(msg, 0x454E414Cu, 4);
            put(msg, c->lanes, 4);
        }
        if (!c->start_tokens.empty()) put(msg, 0x54525453u, 4);  // "STRT": streams cut from given tokens
        if (p.n_seg > 1) {                             // "SEGS": documents ordered arrival by arrival
            put(msg, 0x53474553u, 4);
            put(msg, p.n_seg, 4);
        }
        put(msg, p.T, 4);
        put(msg, p.B, 4);
        put(msg, p.seed, 8);
        put(msg, S, 4);
        put(msg, p.pad_token, 4);
        put(msg, cycle, 4);
        put(msg, U32, 4);
        put(msg, c->checks[0], 8);
        put(msg, c->checks[1], 8);
        const size_t head_bytes = msg.size() - rec_bytes;
        const uint32_t leaves = (S + LEAF - 1) / LEAF;
        if (rec_bytes + head_bytes + 32ull * leaves > c->dig_cap) throw InvalError{"internal: digest buffer"};

        c->timer.begin(PACK_PHASE_CYCLE, c->st);
        const uint32_t zero_err = 0;
        const uint64_t zero_sums[2] = {0, 0};
        if (!p.tabled) up(*c, p.err, &zero_err, 1);
        up(*c, p.cyc_sums, zero_sums, 2);
        up(*c, p.cyc_start, start.data(), S);
        if (p.read_random) up(*c, p.perm_start, ps.data(), S + 1);
        up(*c, c->next_win, nw.data(), S);
        up(*c, c->dig_buf, msg.data(), msg.size());
        up_flush(*c);
        if (p.tabled) dp::launch_cum_slots(p, U32, c->st);
        if (p.read_random) dp::launch_read_order(p, cycle, ps[S], c->st);
        dp::launch_cycle_sums(p, slots, c->next_win, c->stream_next, c->st);  // and each stream's next first token
        uint8_t* const head = c->dig_buf + rec_bytes;
        dp::launch_sha_chunks(c->dig_buf, rec_bytes, REC * LEAF, head + head_bytes, c->st);
        dp::launch_sha_bytes(head, head_bytes + 32ull * leaves, c->dig_buf + c->dig_cap, c->st);
        c->timer.end(c->st);
        h_sums = down(*c, p.cyc_sums, 2);
        const uint64_t* h_next = down(*c, c->stream_next, S);
        const uint8_t* h_digest = down(*c, (const uint8_t*)(c->dig_buf + c->dig_cap), 32);
        const uint32_t* h_cerr = down(*c, p.err, 1);
        sync_staged(*c);
        const uint64_t sums[2] = {h_sums[0], h_sums[1]};
        std::vector<uint64_t> next_tok(h_next, h_next + S);
        uint8_t digest[32];
        std::memcpy(digest, h_digest, 32);
        const uint32_t cerr = *h_cerr;
        reset_staging(*c);
        if (cerr & dp::ERR_INTERNAL) throw InternalError{"internal: a cycle kernel found the plan inconsistent (library bug)"};

        // commit the cycle
        c->U = U32;
        c->cyc_start = start;
        c->taken = taken;
        c->cyc_next = next;
        c->cycle = cycle;
        c->tokens_start = t0;
        c->tokens_next = t0 + slots * p.T;
        c->upd_B = std::move(upd_B);
        c->upd_out0 = std::move(upd_out0);
        c->ready = true;

        if (info) {
            info->cycle = cycle;
            info->n_updates = c->U;
            info->real_tokens = sums[0];
            info->learned_tokens = sums[1];
            info->positions = slots * p.T;
            std::memcpy(info->plan_digest, digest, 32);
            for (uint32_t s = 0; s < S; ++s) {
                const uint64_t M = c->src_win_start[s + 1] - c->src_win_start[s];
                if (info->windows_start) info->windows_start[s] = c->cyc_start[s];
                if (info->windows_taken) info->windows_taken[s] = c->taken[s];
                if (info->windows_remaining) info->windows_remaining[s] = M - c->cyc_start[s] - c->taken[s];
                if (info->kept_docs) info->kept_docs[s] = c->stats[0 * S + s];
                if (info->kept_tokens) info->kept_tokens[s] = c->stats[1 * S + s];
                if (info->held_docs) info->held_docs[s] = c->stats[2 * S + s];
                if (info->held_tokens) info->held_tokens[s] = c->stats[3 * S + s];
                if (info->per_update) info->per_update[s] = c->n_upd[s];
                if (info->stream_next_token) info->stream_next_token[s] = next_tok[s];
            }
        }
        return PACK_OK;
    } catch (const InvalError& e) {
        c->err = e.msg;
        reset_staging(*c);
        return PACK_E_INVAL;
    } catch (const InternalError& e) {
        c->err = e.msg;
        reset_staging(*c);
        return PACK_E_INTERNAL;
    } catch (const dp::HipError& e) {
        reset_staging(*c);
        return fail_hip(c, e);
    } catch (const std::bad_alloc&) {
        c->err = "host allocation failed";
        reset_staging(*c);
        return PACK_E_NOMEM;
    }
}

int pack_status(pack_ctx* c) {
    if (!c) return PACK_E_INVAL;
    c->err.clear();
    try {
        // the staging area is free between calls: every call resets it after its synchronization
        reset_staging(*c);
        const uint32_t* h = d2h_staged(*c, c->p.err_batch, 1);
        DP_HIP(hipStreamSynchronize(c->st));
        const uint32_t e = *h;
        reset_staging(*c);
        if (e & dp::ERR_INTERNAL) {
            dp::launch_zero_u32(c->p.err_batch, 1, c->st);
            DP_HIP(hipStreamSynchronize(c->st));
            c->err = "internal: a batch kernel's bounded wait gave up; the digests of the calls since the last "
                     "pack_status are not valid (library bug)";
            return PACK_E_INTERNAL;
        }
        return PACK_OK;
    } catch (const dp::HipError& e) {
        reset_staging(*c);
        return fail_hip(c, e);
    }
}

int pack_test_option(pack_ctx* c, uint32_t what, uint32_t value) {
    if (!c) return PACK_E_INVAL;
    c->err.clear();
    uint32_t bit = 0;
    switch (what) {
        case PACK_TEST_WAIT_GIVE_UP: bit = dp::TEST_WAIT_GIVE_UP; break;
        case PACK_TEST_CYCLE_FAULT: bit = dp::TEST_CYCLE_FAULT; break;
        case PACK_TEST_SORT_INSERTION: bit = dp::TEST_SORT_INSERTION; break;
        case PACK_TEST_DIGEST_SLICES: bit = dp::TEST_DIGEST_SLICES; break;
        default: c->err = "unknown test option"; return PACK_E_INVAL;
    }
    if (value) c->p.test_opts |= bit;
    else c->p.test_opts &= ~bit;
    return PACK_OK;
}

int pack_batch(pack_ctx* c, uint32_t step, uint32_t n_steps, const pack_out* out) {
    if (!c) return PACK_E_INVAL;
    c->err.clear();
    if (!c->ready) {
        c->err = "no cycle planned (or the last pack_cycle failed)";
        return PACK_E_STATE;
    }
    if (n_steps == 0 || (uint64_t)step + n_steps > c->U) {
        c->err = "step range outside the current cycle";
        return PACK_E_RANGE;
    }
    if (!out || !out->tokens || !out->pos || !out->doc || !out->mask) {
        c->err = "tokens, pos, doc and mask outputs are required";
        return PACK_E_INVAL;
    }
    if (((uintptr_t)out->tokens | (uintptr_t)out->pos | (uintptr_t)out->doc | (uintptr_t)out->digests) % 16 ||
        (uintptr_t)out->mask % 4 || (uintptr_t)out->learned % 8) {
        c->err = "outputs must be 16-byte aligned (mask 4-byte, learned 8-byte)";
        return PACK_E_INVAL;
    }
    try {
        dp::EmitArgs a{};
        a.tok = out->tokens;
        a.pos = out->pos;
        a.doc = out->doc;
        a.mask = out->mask;
        a.learned = out->learned;
        a.digests = out->digests;
        a.step = step;
        a.n_steps = n_steps;
        a.rank = c->cfg.rank;
        a.per = c->p.B / c->cfg.world;
        a.n_out = c->p.ramp ? c->upd_out0[step + n_steps] - c->upd_out0[step] : (uint64_t)n_steps * a.per;
        if ((uint64_t)n_steps * a.per >= (1ull << 31)) {
            c->err = "too many windows in one call";
            return PACK_E_RANGE;
        }
        if (a.digests) {  // emission beside the digests, one kernel
            c->timer.begin(PACK_PHASE_DIGEST, c->st);
            dp::launch_emit_sha(c->p, a, c->st);
            c->timer.end(c->st);
        } else {
            c->timer.begin(PACK_PHASE_EMIT, c->st);
            dp::launch_emit(c->p, a, c->st);
            c->timer.end(c->st);
        }
        if (a.learned) {
            c->timer.begin(PACK_PHASE_LEARNED, c->st);
            dp::launch_learned(c->p, a, c->st);
            c->timer.end(c->st);
        }
        return PACK_OK;
    } catch (const dp::HipError& e) {
        return fail_hip(c, e);
    }
}

int pack_batch_packed(pack_ctx* c, uint32_t step, uint32_t n_steps, const pack_out_packed* out) {
    if (!c) return PACK_E_INVAL;
    c->err.clear();
    if (!c->ready) {
        c->err = "no cycle planned (or the last pack_cycle failed)";
        return PACK_E_STATE;
    }
    if (n_steps == 0 || (uint64_t)step + n_steps > c->U) {
        c->err = "step range outside the current cycle";
        return PACK_E_RANGE;
    }
    if (!out || !out->tokens || !out->pos || !out->doc || !out->mask || !out->row_start || !out->length) {
        c->err = "tokens, pos, doc, mask, row_start and length outputs are required";
        return PACK_E_INVAL;
    }
    if (((uintptr_t)out->tokens | (uintptr_t)out->pos | (uintptr_t)out->doc) % 16 || (uintptr_t)out->mask % 4 ||
        ((uintptr_t)out->row_start | (uintptr_t)out->length | (uintptr_t)out->learned) % 8) {
        c->err = "tokens/pos/doc must be 16-byte aligned, mask 4-byte, row_start/length/learned 8-byte aligned";
        return PACK_E_INVAL;
    }
    try {
        dp::EmitArgs a{};
        a.tok = out->tokens;
        a.pos = out->pos;
        a.doc = out->doc;
        a.mask = out->mask;
        a.learned = out->learned;
        a.row_start = out->row_start;
        a.length = out->length;
        a.bucket = out->bucket;
        a.step = step;
        a.n_steps = n_steps;
        a.rank = c->cfg.rank;
        a.per = c->p.B / c->cfg.world;
        a.n_out = c->p.ramp ? c->upd_out0[step + n_steps] - c->upd_out0[step] : (uint64_t)n_steps * a.per;
        if ((uint64_t)n_steps * a.per >= (1ull << 31)) {
            c->err = "too many windows in one call";
            return PACK_E_RANGE;
        }
        c->timer.begin(PACK_PHASE_EMIT, c->st);
        dp::launch_emit_packed(c->p, a, c->st);
        c->timer.end(c->st);
        if (a.learned) {
            c->timer.begin(PACK_PHASE_LEARNED, c->st);
            dp::launch_learned(c->p, a, c->st);
            c->timer.end(c->st);
        }
        return PACK_OK;
    } catch (const dp::HipError& e) {
        return fail_hip(c, e);
    }
}

int pack_fingerprint(pack_ctx* c, const uint8_t* digests, uint32_t n_batches, uint8_t* out) {
    if (!c) return PACK_E_INVAL;
    c->err.clear();
    if (!digests || !out) {
        c->err = "digests and out are required";
        return PACK_E_INVAL;
    }
    if ((uintptr_t)digests % 4) {
        c->err = "digests must be 4-byte aligned";
        return PACK_E_INVAL;
    }
    if (c->p.ramp) {
        c->err = "batches of a ramp differ in size: use pack_fingerprint_steps";
        return PACK_E_STATE;
    }
    if (n_batches == 0) return PACK_OK;
    try {
        c->timer.begin(PACK_PHASE_FINGERPRINT, c->st);
        dp::launch_batch_fp(digests, c->p.B, n_batches, out, c->st);
        c->timer.end(c->st);
        return PACK_OK;
    } catch (const dp::HipError& e) {
        return fail_hip(c, e);
    }
}

int pack_fingerprint_steps(pack_ctx* c, uint32_t step, uint32_t n_steps, const uint8_t* digests, uint8_t* out) {
    if (!c) return PACK_E_INVAL;
    c->err.clear();
    if (!digests || !out) {
        c->err = "digests and out are required";
        return PACK_E_INVAL;
    }
    if ((uintptr_t)digests % 4) {
        c->err = "digests must be 4-byte aligned";
        return PACK_E_INVAL;
    }
    if (!c->ready) {
        c->err = "no cycle planned (or the last pack_cycle failed)";
        return PACK_E_STATE;
    }
    if ((uint64_t)step + n_steps > c->U) {
        c->err = "step range outside the current cycle";
        return PACK_E_RANGE;
    }
    if (n_steps == 0) return PACK_OK;
    try {
        c->timer.begin(PACK_PHASE_FINGERPRINT, c->st);
        if (c->p.ramp) dp::launch_batch_fp_var(digests, c->p.upd_slot0, step, n_steps, out, c->st);
        else dp::launch_batch_fp(digests, c->p.B, n_steps, out, c->st);
        c->timer.end(c->st);
        return PACK_OK;
    } catch (const dp::HipError& e) {
        return fail_hip(c, e);
    }
}

int pack_inspect(const pack_ctx* cc, uint32_t what, void* host_dst, uint64_t capacity, uint64_t* needed) {
    if (!cc) return PACK_E_INVAL;
    pack_ctx* c = const_cast<pack_ctx*>(cc);
    const dp::Plan& p = c->p;
    const void* src = nullptr;
    uint64_t count = 0;
    int width = 0;      // bytes per element on the device
    int out_width = 0;  // bytes per element in the host copy
    switch (what) {
        case PACK_INSPECT_HASH: src = p.hash; count = p.n_docs; width = out_width = 8; break;
        case PACK_INSPECT_KEEP: src = p.keep; count = p.n_docs; width = out_width = 1; break;
        case PACK_INSPECT_ORDER: src = p.order; count = p.n_kept; width = out_width = 4; break;
        case PACK_INSPECT_SRC_DOC_START: src = p.src_doc_start; count = p.S + 1; width = out_width = 8; break;
        case PACK_INSPECT_PIECE_DOC: src = p.pc_doc; count = p.n_pieces; width = out_width = 4; break;
        case PACK_INSPECT_PIECE_OFF: src = p.pc_off; count = p.n_pieces; width = out_width = 4; break;
        case PACK_INSPECT_PIECE_LEN: src = p.pc_len; count = p.n_pieces; width = out_width = 4; break;
        case PACK_INSPECT_PIECE_WOFF: src = p.pc_woff; count = p.n_pieces; width = out_width = 4; break;
        case PACK_INSPECT_SRC_PIECE_START: src = p.src_piece_start; count = p.S + 1; width = out_width = 8; break;
        case PACK_INSPECT_WIN_FIRST: src = p.win_first; count = p.n_windows + 1; width = 4; out_width = 8; break;
        case PACK_INSPECT_SRC_WIN_START: src = p.src_win_start; count = p.S + 1; width = out_width = 8; break;
        case PACK_INSPECT_WIN_REAL: src = p.win_real; count = p.n_windows; width = 4; out_width = 8; break;
        case PACK_INSPECT_WIN_LEARN: src = p.win_learn; count = p.n_windows; width = 4; out_width = 8; break;
        case PACK_INSPECT_PER_UPDATE: src = p.n_upd; count = p.S; width = out_width = 4; break;
        case PACK_INSPECT_SLOT_SRC: src = p.slot_src; count = p.B; width = out_width = 4; break;
        case PACK_INSPECT_SLOT_K: src = p.slot_k; count = p.B; width = out_width = 4; break;
        case PACK_INSPECT_COUNTS: count = 3; width = out_width = 8; break;
        case PACK_INSPECT_UPDATE_BATCH:
            if (!c->ready) {
                c->err = "no cycle planned (or the last pack_cycle failed)";
                return PACK_E_STATE;
            }
            count = c->U;
            width = out_width = 4;
            break;
        case PACK_INSPECT_CUM_TAKEN:
            if (!p.tabled || !c->ready) {
                c->err = "no per-update schedule: neither PACK_FLAG_CUMULATIVE nor a ramp, or no cycle yet";
                return PACK_E_STATE;
            }
            src = p.cum_A;
            count = ((uint64_t)c->U + 1) * p.S;
            width = out_width = 4;
            break;
        default: c->err = "unknown inspect code"; return PACK_E_INVAL;
    }
    const uint64_t bytes = count * out_width;
    if (needed) *needed = bytes;
    if (capacity < bytes) return PACK_E_RANGE;
    if (!host_dst && bytes) return PACK_E_INVAL;
    try {
        if (what == PACK_INSPECT_COUNTS) {
            uint64_t v[3] = {p.n_kept, p.n_pieces, p.n_windows};
            std::memcpy(host_dst, v, sizeof v);
            return PACK_OK;
        }
        if (what == PACK_INSPECT_UPDATE_BATCH) {  // host copy of the cycle's batches
            uint32_t* o = static_cast<uint32_t*>(host_dst);
            for (uint64_t u = 0; u < count; ++u) o[u] = p.ramp ? c->upd_B[u] : p.B;
            return PACK_OK;
        }
        if (width == out_width) {
            if (bytes) DP_HIP(hipMemcpyAsync(host_dst, src, bytes, hipMemcpyDeviceToHost, c->st));
            DP_HIP(hipStreamSynchronize(c->st));
        } else {
            std::vector<uint32_t> tmp(count);
            if (count) DP_HIP(hipMemcpyAsync(tmp.data(), src, count * 4, hipMemcpyDeviceToHost, c->st));
            DP_HIP(hipStreamSynchronize(c->st));
            uint64_t* o = static_cast<uint64_t*>(host_dst);
            for (uint64_t i = 0; i < count; ++i) o[i] = tmp[i];
        }
        return PACK_OK;
    } catch (const dp::HipError& e) {
        return fail_hip(c, e);
    }
}

int pack_get_timings(pack_ctx* c, pack_timings* out, int reset) {
    if (!c || !out) return PACK_E_INVAL;
    try {
        DP_HIP(hipStreamSynchronize(c->st));
        c->timer.resolve();
        for (int i = 0; i < PACK_N_PHASES; ++i) {
            out->ms[i] = c->timer.ms[i];
            out->calls[i] = c->timer.calls[i];
            if (reset) {
                c->timer.ms[i] = 0;
                c->timer.calls[i] = 0;
            }
        }
        return PACK_OK;
    } catch (const dp::HipError& e) {
        return fail_hip(c, e);
    }
}

void pack_destroy(pack_ctx* c) { release(c); }

}  // extern "C"
