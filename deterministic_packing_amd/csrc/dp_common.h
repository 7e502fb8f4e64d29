// dp_common.h — device primitives and the plan workspace shared by the
// library's HIP translation units.  Written for gfx950 (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dp {

constexpr int WAVE = 64;
constexpr uint32_t END = 0xFFFFFFFFu;  // "past the end of the source" in jump tables
// error bit set by a kernel that finds the plan inconsistent (a library bug)
// or whose bounded wait gives up: the access is skipped and the calling
// function (pack_init, pack_cycle) or pack_status reports PACK_E_INTERNAL
constexpr uint32_t ERR_INTERNAL = 0x100u;
// test options (the PACK_TEST_* values of dpack.h)
constexpr uint32_t TEST_WAIT_GIVE_UP = 1u;
constexpr uint32_t TEST_CYCLE_FAULT = 2u;
constexpr uint32_t TEST_SORT_INSERTION = 4u;
constexpr uint32_t TEST_DIGEST_SLICES = 8u;

// ---------------------------------------------------------------- errors
struct HipError {
    hipError_t code;
    const char* what;
};

#define DP_HIP(call)                                                    \
    do {                                                                \
        hipError_t e_ = (call);                                         \
        if (e_ != hipSuccess) throw ::dp::HipError{e_, #call};          \
    } while (0)

// ---------------------------------------------------------------- hashing primitives

// SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014).
__host__ __device__ inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

constexpr uint32_t PHI32 = 0x9E3779B1u;
constexpr uint64_t PHI64 = 0x9E3779B97F4A7C15ull;

// Philox4x32-10 (Salmon, Moraes, Dror & Shaw, SC'11).  Returns the first two
// output words as x1·2^32 + x0, which is all the shuffle key needs.
__device__ inline uint64_t philox_key64(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                        uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return ((uint64_t)c1 << 32) | c0;
}

// 128-bit compare of a·b against c·d for 64-bit operands: -1, 0, +1.
__host__ __device__ inline int cmp_mul128(uint64_t a, uint64_t b, uint64_t c, uint64_t d) {
    const unsigned __int128 x = (unsigned __int128)a * b;
    const unsigned __int128 y = (unsigned __int128)c * d;
    return x < y ? -1 : (x > y ? 1 : 0);
}

// ---------------------------------------------------------------- wave helpers
// Cross-lane moves by DPP, in registers (no LDS crossbar): row_shr:n (lane i
// reads lane i − n of its row of 16), row_bcast:15 / row_bcast:31 (lane 15 /
// 31 to the next row / rows), wave_shr:1 (lane i reads lane i − 1),
// wave_shl:1 (lane i reads lane i + 1).  A lane whose source lies outside the
// pattern, or whose row is masked off, keeps `old`.  Every lane of the
// wavefront must be active.
enum : int {
    DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118,
    DPP_WAVE_SHL1 = 0x130, DPP_WAVE_SHR1 = 0x138, DPP_BCAST15 = 0x142, DPP_BCAST31 = 0x143,
};

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp32(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xF, false);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp64(uint64_t old, uint64_t v) {
    const uint32_t lo = dpp32<CTRL, ROWS>((uint32_t)old, (uint32_t)v);
    const uint32_t hi = dpp32<CTRL, ROWS>((uint32_t)(old >> 32), (uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive sum over lanes 0 .. l, in lane l: within rows of 16 by shifts of
// 1, 2, 4, 8, then row 0's total into row 1 and row 2's into row 3, then
// lane 31's into rows 2 and 3.  Every lane must be active.
__device__ __forceinline__ uint64_t wave_incl_u64(uint64_t v) {
    v += dpp64<DPP_ROW_SHR1, 0xF>(0, v);
    v += dpp64<DPP_ROW_SHR2, 0xF>(0, v);
    v += dpp64<DPP_ROW_SHR4, 0xF>(0, v);
    v += dpp64<DPP_ROW_SHR8, 0xF>(0, v);
    v += dpp64<DPP_BCAST15, 0xA>(0, v);
    v += dpp64<DPP_BCAST31, 0xC>(0, v);
    return v;
}

__device__ __forceinline__ uint32_t wave_incl_u32(uint32_t v) {
    v += dpp32<DPP_ROW_SHR1, 0xF>(0, v);
    v += dpp32<DPP_ROW_SHR2, 0xF>(0, v);
    v += dpp32<DPP_ROW_SHR4, 0xF>(0, v);
    v += dpp32<DPP_ROW_SHR8, 0xF>(0, v);
    v += dpp32<DPP_BCAST15, 0xA>(0, v);
    v += dpp32<DPP_BCAST31, 0xC>(0, v);
    return v;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, uint32_t k) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, (int)k);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), (int)k);
    return ((uint64_t)hi << 32) | lo;
}

// The sum of v over the wavefront, in every lane.  Every lane must be active.
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) { return readlane64(wave_incl_u64(v), WAVE - 1); }

__device__ inline uint32_t lane_id() { return __lane_id(); }

// ---------------------------------------------------------------- plan workspace
// Device arrays of the plan; sizes in the comments (D docs, K kept, P pieces,
// M windows, S sources, G groups, L lifting levels).
// A span of the batch-size ramp: from update `first` of the cycle on, B windows
// per update, slot0 seats before it (the next span's first update ends it).
struct RampSpan {
    uint64_t first;  // first update of the span in the cycle
    uint64_t slot0;  // its first slot
    uint64_t out0;   // its first output window of this rank
    uint32_t B;      // windows per update in the span
    uint32_t k;      // ramp piece
};

// Workspace of the single-pass scans: a tile ticket (zero between scans) and
// one status word per tile: state (bits 63..62: 1 the tile's sum, 2 its
// inclusive prefix), the scan's epoch (61..40; words of other epochs count as
// nothing published) and the value (39..0), in one word so that a relaxed
// device-scope atomic load sees value and state together (no fence, which
// would write back the whole L2 of the publishing XCD).  err receives
// ERR_INTERNAL if a look-back's bounded wait gives up.  epoch (host) is the
// last epoch used; at its wrap the workspace is zeroed again.
struct ScanWs {
    uint32_t* ticket;
    uint64_t* status;
    uint32_t* err;
    uint32_t* epoch;  // host
    uint64_t words;   // 32-bit words of the workspace, ticket first
};
constexpr uint64_t SCAN_VALUE_BITS = 40;  // scanned totals stay below 2^40 (n_tokens < 2^40)

struct Plan {
    // inputs (borrowed)
    const uint32_t* tokens;
    const uint64_t* offsets;
    const uint16_t* source;
    const uint16_t* stratum;      // may be null
    const uint32_t* prompt_len;   // may be null
    const uint16_t* segment;      // may be null: the arrival of each document (n_seg > 1)
    uint32_t n_seg;               // arrivals (1: none); groups are (stream, arrival, stratum)
    uint64_t n_tokens, n_docs;
    uint32_t S, G, T, B;
    uint64_t seed;
    uint32_t pad_token;
    uint32_t wrap;                // 1: wrap packing (cut every T tokens), 0: next-fit
    uint32_t heldout;             // 1: the stream is the held-out documents (validation)
    uint32_t read_random;         // 1: each cycle's windows of a source are read in a random order
    uint32_t cumulative;          // 1: per-update counts from the cycle's cumulative quotas
    uint32_t ramp;                // 1: batch-size ramp (each update has its own batch)
    uint32_t tabled;              // cumulative or ramp: windows looked up in per-update slot tables
    uint32_t world;               // ranks sharing each update's slots
    uint32_t lanes;               // lanes L (1: none); streams s·L + l, the schedule per lane over B/L seats
    uint32_t S_real;              // the recipe's sources (S = S_real·lanes streams)
    uint32_t digest_chunked;      // 1: window digests over the digests of 4,096-byte chunks of the record
    uint32_t* chunk_cd;           // digest_chunked: the chunk digests of one slice of windows (8 words each)
    uint64_t chunk_cd_words;      // its size in words

    // recipe on device
    uint32_t* gbase;              // [S·n_seg+1] first group of each (stream, arrival)
    uint32_t* n_strata;           // [S]
    uint64_t* weight;             // [S]
    uint32_t* bp;                 // [S]

    // A1/A2
    uint32_t* group;              // [D] group of each doc
    uint64_t* hash;               // [D]
    uint8_t* keep;                // [D]
    uint32_t* kept_pos;           // [D+1] exclusive scan of keep
    uint64_t* stats;              // [4][S] kept docs, kept tokens, held docs, held tokens
    uint32_t* err;                // [1] validation and plan/cycle error flags (cleared by each synchronous call)
    uint32_t* err_batch;          // [1] error flags of the asynchronous batch kernels (cleared by pack_status)
    uint32_t test_opts;           // test options (PACK_TEST_*): 0 in normal use

    // A3 sort
    uint64_t* key[2];             // [D]
    uint32_t* val[2];             // [D]
    uint32_t* hist;               // sort workspace
    ScanWs scan;                  // single-pass scan workspace
    uint32_t sort_buf;            // which buffer holds the sorted result

    // A4
    uint32_t* group_start;        // [G+1]
    uint64_t* gpre;               // [D+1] length prefix in sorted order
    uint32_t* order;              // [D] merged order (kept docs)
    uint64_t* src_doc_start;      // [S+1]

    // A5
    uint32_t* piece_start;        // [D+1] exclusive scan of piece counts over the order
    uint64_t* opre;               // [D+1] length prefix over the order
    uint32_t* pc_doc;             // [P]
    uint32_t* pc_off;             // [P]
    uint32_t* pc_len;             // [P]
    uint32_t* pc_woff;            // [P]
    uint4* pc_emit;               // [P] emission view: (u64 token index of window position 0, doc, mask start)
    uint32_t* pad16;              // [16] the pad token, 16 times (a load source for padding)
    uint64_t* pc_pre;             // [P+1] token prefix over pieces
    uint64_t* src_piece_start;    // [S+1]
    uint32_t* jump;               // [L][P] lifting table
    uint32_t levels;
    uint64_t* src_win_start;      // [S+1]
    uint32_t* win_first;          // [M+1]
    uint32_t* win_real;           // [M]
    uint32_t* win_learn;          // [M]

    // A6
    uint32_t* n_upd;              // [S]
    uint32_t* slot_src;           // [B]
    uint32_t* slot_k;             // [B]
    uint64_t* cyc_start;          // [S] first window of the current cycle per source
    uint64_t* checks;             // [2] order check, hash check
    uint64_t* cyc_sums;           // [2] real, learned over the current cycle
    // random read order (read_random): per cycle, source s reads its i-th cycle
    // window from position perm[perm_start[s] + i] of its cycle range
    uint64_t* perm_start;         // [S+1]
    uint32_t* perm;               // [U·B]
    uint64_t* wkey[2];            // sort workspace [cap windows]
    uint32_t* wval[2];
    uint32_t* wgroup;
    // cumulative mixture (cumulative): windows of each source taken before each
    // update, and every update's slot table as (source, cycle window index)
    uint32_t* cum_A;              // [(U_cap+1)·S]
    uint64_t* cum_rem;            // [S] windows each source has left at the cycle start
    uint64_t* cum_out;            // [S+1] windows taken per source, then U
    uint32_t* cslot_src;          // [slots of the cycle ≤ P]
    uint32_t* cslot_i;            // [slots of the cycle ≤ P]
    // batch-size ramp: per update of the cycle (U_cap+1 entries)
    uint32_t* upd_B;              // windows of the update (all ranks)
    uint64_t* upd_slot0;          // first slot of the update in the cycle (prefix of upd_B)
    uint64_t* upd_out0;           // first of this rank's output windows (prefix of upd_B/world)
    const struct RampSpan* spans; // the ramp's pieces from the cycle's first update on (the last without end)
    const uint64_t* start_tok;    // [S] first token of each stream to cut, or null (from the stream's start)
    uint32_t n_spans;

    // sizes known after the corresponding step (host copies)
    uint64_t n_kept, n_pieces, n_windows;
    uint64_t cap_pieces;          // allocation bound for pieces
    // while pack_init runs, the piece and window counts stay on the device
    // (n_pieces and n_windows then hold the bound cap_pieces); null afterwards
    const uint32_t* n_pieces_dev;
    const uint64_t* n_windows_dev;
};

// the plan's piece and window counts (from the device while pack_init runs),
// never above the allocation bound
__device__ inline uint64_t plan_pieces(const Plan& p) {
    const uint64_t n = p.n_pieces_dev ? *p.n_pieces_dev : p.n_pieces;
    return n < p.cap_pieces ? n : p.cap_pieces;
}
__device__ inline uint64_t plan_windows(const Plan& p) {
    const uint64_t n = p.n_windows_dev ? *p.n_windows_dev : p.n_windows;
    return n < p.cap_pieces ? n : p.cap_pieces;
}

// Global window index of slot j of update b of the current cycle: source s
// = slot_src[j] contributes its (slot_k[j])-th window of the update, i.e. its
// i-th window of the cycle, i = b·n_s + slot_k[j] (with the cumulative
// mixture, s and i come from update b's own slot table): window
// cyc_start[s] + i of its stream, or cyc_start[s] + perm[perm_start[s] + i]
// with the random read order.
__device__ inline uint64_t window_of_slot(const Plan& p, uint64_t x) {  // slot x of a tabled cycle
    const uint32_t s = p.cslot_src[x];
    uint64_t i = p.cslot_i[x];
    if (p.read_random) i = p.perm[p.perm_start[s] + i];
    return p.src_win_start[s] + p.cyc_start[s] + i;
}

__device__ inline uint64_t window_of(const Plan& p, uint64_t b, uint32_t j) {
    if (p.tabled) return window_of_slot(p, (p.ramp ? p.upd_slot0[b] : b * p.B) + j);
    const uint32_t s = p.slot_src[j];
    uint64_t i = b * p.n_upd[s] + p.slot_k[j];  // the source's i-th window of the cycle
    if (p.read_random) i = p.perm[p.perm_start[s] + i];
    return p.src_win_start[s] + p.cyc_start[s] + i;
}

// ---------------------------------------------------------------- SHA-256 (FIPS 180-4)
__host__ __device__ inline uint32_t sha_k(int t) {
    constexpr uint32_t K[64] = {
        0x428a2f98u, 0x71374491u, 0xb5c0fbcfu, 0xe9b5dba5u, 0x3956c25bu, 0x59f111f1u, 0x923f82a4u, 0xab1c5ed5u,
        0xd807aa98u, 0x12835b01u, 0x243185beu, 0x550c7dc3u, 0x72be5d74u, 0x80deb1feu, 0x9bdc06a7u, 0xc19bf174u,
        0xe49b69c1u, 0xefbe4786u, 0x0fc19dc6u, 0x240ca1ccu, 0x2de92c6fu, 0x4a7484aau, 0x5cb0a9dcu, 0x76f988dau,
        0x983e5152u, 0xa831c66du, 0xb00327c8u, 0xbf597fc7u, 0xc6e00bf3u, 0xd5a79147u, 0x06ca6351u, 0x14292967u,
        0x27b70a85u, 0x2e1b2138u, 0x4d2c6dfcu, 0x53380d13u, 0x650a7354u, 0x766a0abbu, 0x81c2c92eu, 0x92722c85u,
        0xa2bfe8a1u, 0xa81a664bu, 0xc24b8b70u, 0xc76c51a3u, 0xd192e819u, 0xd6990624u, 0xf40e3585u, 0x106aa070u,
        0x19a4c116u, 0x1e376c08u, 0x2748774cu, 0x34b0bcb5u, 0x391c0cb3u, 0x4ed8aa4au, 0x5b9cca4fu, 0x682e6ff3u,
        0x748f82eeu, 0x78a5636fu, 0x84c87814u, 0x8cc70208u, 0x90befffau, 0xa4506cebu, 0xbef9a3f7u, 0xc67178f2u};
    return K[t];
}

__device__ inline uint32_t rotr32(uint32_t x, uint32_t n) { return __builtin_amdgcn_alignbit(x, x, n); }

// One compression of a 64-byte block given as 16 big-endian words.  On
// gfx950 the rotates map to v_alignbit_b32, the 3-input xors, Ch and Maj to
// v_bitop3_b32, and the sums to v_add3_u32.
__device__ inline void sha256_compress(uint32_t H[8], uint32_t W[16]) {
    uint32_t a = H[0], b = H[1], c = H[2], d = H[3], e = H[4], f = H[5], g = H[6], h = H[7];
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
        const uint32_t S1 = __builtin_amdgcn_bitop3_b32(rotr32(e, 6), rotr32(e, 11), rotr32(e, 25), 0x96);
        const uint32_t ch = __builtin_amdgcn_bitop3_b32(e, f, g, 0xCA);   // (e & f) | (~e & g)
        const uint32_t T1 = h + S1 + ch + sha_k(t) + w;
        const uint32_t S0 = __builtin_amdgcn_bitop3_b32(rotr32(a, 2), rotr32(a, 13), rotr32(a, 22), 0x96);
        const uint32_t mj = __builtin_amdgcn_bitop3_b32(a, b, c, 0xE8);   // majority
        h = g; g = f; f = e; e = d + T1;
        d = c; c = b; b = a; a = T1 + S0 + mj;
    }
    H[0] += a; H[1] += b; H[2] += c; H[3] += d;
    H[4] += e; H[5] += f; H[6] += g; H[7] += h;
}

__device__ inline void sha256_init(uint32_t H[8]) {
    H[0] = 0x6a09e667u; H[1] = 0xbb67ae85u; H[2] = 0x3c6ef372u; H[3] = 0xa54ff53au;
    H[4] = 0x510e527fu; H[5] = 0x9b05688cu; H[6] = 0x1f83d9abu; H[7] = 0x5be0cd19u;
}

__device__ inline uint32_t bswap32(uint32_t x) { return __builtin_bswap32(x); }

// ---------------------------------------------------------------- launchers
// (each defined in the translation unit that holds the kernels)
void launch_validate(const Plan& p, uint64_t* S, uint32_t* first, hipStream_t st);  // also zeroes S, fills first
void launch_hash(const Plan& p, uint64_t* S, uint32_t* first, hipStream_t st);
uint64_t hash_tile_count(uint64_t n_tokens);
void launch_keep_scan(Plan& p, hipStream_t st);       // kept_pos + compaction into val[0], keys, group counts
void launch_sort(Plan& p, hipStream_t st);            // by (group, key64, d); sets sort_buf
// counted: the workspace's first sort_count_words(n, G) words were zeroed and
// its first G hold each group's element count (else the sort does both)
uint32_t sort_pairs(uint64_t* const key[2], uint32_t* const val[2], const uint32_t* group, uint64_t n, uint32_t G,
                    uint32_t* hist_ws, const ScanWs& scan, uint32_t test_opts, bool counted, hipStream_t st);
uint64_t sort_count_words(uint64_t n, uint64_t G);  // group and bucket counts of a sort of n pairs
void launch_read_order(Plan& p, uint32_t cycle, uint64_t total, hipStream_t st);  // perm of each source's cycle windows
void launch_merge(Plan& p, hipStream_t st);           // group_start, gpre, order, src_doc_start
void launch_piece_count(Plan& p, hipStream_t st);     // piece_start, opre
void launch_pieces(Plan& p, hipStream_t st);          // piece table, pc_pre, src_piece_start
void launch_lifting(Plan& p, hipStream_t st);         // jump tables
void launch_window_count(Plan& p, hipStream_t st);    // src_win_start
void launch_windows(Plan& p, hipStream_t st);         // win_first, pc_woff, win_real, win_learn
void launch_mixture_w(Plan& p, uint64_t W, uint32_t* nstart, hipStream_t st);  // n_upd, slot table
void launch_apportion(Plan& p, uint64_t W, uint32_t B, uint32_t* n_out, hipStream_t st);  // n_s of a batch B
void launch_zero_u32(uint32_t* a, uint64_t n, hipStream_t st);
void launch_fill_u32(uint32_t* a, uint64_t n, uint32_t v, hipStream_t st);

// up to XFER_MAX device-to-device copies of small ranges in one launch (the
// host's uploads and downloads pass through a contiguous mailbox, so a batch of
// them costs one copy and this kernel); pointers 4-byte aligned
constexpr uint32_t XFER_MAX = 16;
struct Xfer {
    const uint8_t* src;
    uint8_t* dst;
    uint64_t bytes;
};
struct XferList {
    Xfer x[XFER_MAX];
    uint32_t n;
};
void launch_xfer(const XferList& l, hipStream_t st);
uint64_t sort_hist_words(uint64_t n, uint64_t G);
void launch_checks(Plan& p, hipStream_t st);          // order / hash checks
// the cycle's real and learned sums into cyc_sums (zeroed before), and each
// stream's first token of the window next_win[s] (~0: the stream's total)
void launch_cycle_sums(Plan& p, uint64_t total_slots, const uint64_t* next_win, uint64_t* stream_next,
                       hipStream_t st);
// cumulative mixture of a cycle: the schedule (cum_A, cum_out), then, once the
// host has accepted U, every update's slot table.  integral: every update's
// seats times every weight is a multiple of W (the schedule has a closed form)
void launch_cumulative(Plan& p, uint64_t W, uint64_t cap, bool integral, hipStream_t st);
void launch_cum_slots(Plan& p, uint32_t U, hipStream_t st);
// lanes: stream ids of the documents, one lane's counts/slots to every lane, one lane's schedule to every lane
void launch_lane_source(const uint16_t* source, uint64_t n_docs, uint32_t S_real, uint32_t L, uint16_t* out,
                        hipStream_t st);
void launch_lane_expand(Plan& p, const uint32_t* n_real, const uint32_t* lane_src, const uint32_t* lane_k,
                        hipStream_t st);
void launch_cum_expand(Plan& p, const uint32_t* cum_Ar, uint64_t U, hipStream_t st);
// batch-size ramp: piece spans of a cycle (host-computed) → per-update tables (RampSpan above)
void launch_ramp_fill(Plan& p, const RampSpan* spans, uint32_t n_spans, uint64_t n_upd, hipStream_t st);
// fixed apportionment with a ramp: cum_A[u][s] = Σ over spans of whole updates before u · n_s of the span's piece
void launch_ramp_fixed_A(Plan& p, const RampSpan* spans, uint32_t n_spans, const uint32_t* ramp_n, uint64_t U,
                         hipStream_t st);

struct EmitArgs {
    uint32_t* tok; int32_t* pos; int32_t* doc; uint8_t* mask;
    int64_t* learned; uint8_t* digests;
    uint32_t step, n_steps, rank, per;  // per: B/world, the largest batch's windows per rank
    uint64_t n_out;                     // this rank's windows of the call
    int64_t* row_start; int64_t* length; uint32_t bucket;  // padding-free rows only
};

// Output window w of a call: update a.step + i, this rank's window jj of it,
// and the rank's windows of that update (B_b/world with a ramp).
__device__ inline uint64_t out_window(const Plan& p, const EmitArgs& a, uint64_t w, uint32_t* i_out,
                                      uint32_t* jj_out, uint32_t* per_out) {
    uint32_t i, jj, per;
    if (!p.ramp) {  // a launch's window index fits 32 bits: 32-bit division
        i = (uint32_t)w / a.per;
        jj = (uint32_t)w - i * a.per;
        per = a.per;
    } else {
        const uint64_t e = p.upd_out0[a.step] + w;
        uint32_t lo = a.step, hi = a.step + a.n_steps;  // upd_out0[lo] ≤ e < upd_out0[hi]
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            if (p.upd_out0[mid] <= e) lo = mid;
            else hi = mid;
        }
        i = lo - a.step;
        jj = (uint32_t)(e - p.upd_out0[lo]);
        per = (uint32_t)(p.upd_out0[lo + 1] - p.upd_out0[lo]);
    }
    *i_out = i;
    *jj_out = jj;
    *per_out = per;
    return window_of(p, (uint64_t)a.step + i, a.rank * per + jj);
}

// this rank's windows of update a.step + i
__device__ inline uint32_t out_per(const Plan& p, const EmitArgs& a, uint32_t i) {
    return p.ramp ? (uint32_t)(p.upd_out0[a.step + i + 1] - p.upd_out0[a.step + i]) : a.per;
}
void launch_emit(const Plan& p, const EmitArgs& a, hipStream_t st);
void launch_emit_packed(const Plan& p, const EmitArgs& a, hipStream_t st);  // padding-free rows
void launch_learned(const Plan& p, const EmitArgs& a, hipStream_t st);
// chunked window digests: chunks of DIGEST_CHUNK bytes of a window's 13·T-byte record
constexpr uint32_t DIGEST_CHUNK = 4096;
__host__ __device__ inline uint64_t digest_chunks(uint64_t T) { return (13 * T + DIGEST_CHUNK - 1) / DIGEST_CHUNK; }
void launch_emit_sha(const Plan& p, const EmitArgs& a, hipStream_t st);  // emission and window digests
uint64_t chunk_slice_windows(const Plan& p);  // chunked digests: windows of one slice of the scratch
void launch_chunk_hash(const Plan& p, const EmitArgs& a, uint64_t w0, uint64_t nw, hipStream_t st);
void launch_batch_fp(const uint8_t* digests, uint32_t B, uint32_t n_batches, uint8_t* out, hipStream_t st);
// batches of B_b digests: batch b covers digests [slot0[step+b] − slot0[step], slot0[step+b+1] − slot0[step])
void launch_batch_fp_var(const uint8_t* digests, const uint64_t* slot0, uint32_t step, uint32_t n_batches,
                         uint8_t* out, hipStream_t st);
void launch_sha_chunks(const uint8_t* msg, uint64_t len, uint32_t chunk, uint8_t* out, hipStream_t st);
void launch_sha_bytes(const uint8_t* msg, uint64_t len, uint8_t* out, hipStream_t st);

// scans (scan.hip): single pass, tiles in ticket order, each tile's prefix
// from its predecessors' published aggregates (decoupled look-back)
uint64_t scan_ws_tiles(uint64_t n_max);          // tiles of the largest scan
size_t scan_ws_bytes(uint64_t n_max);            // workspace bytes for scans of up to n_max items
ScanWs scan_ws_at(void* base, uint64_t n_max, uint32_t* err, uint32_t* host_epoch);  // zeroed by the caller once, epoch 0
// exclusive scans writing out[0..n] (out[n] = total)
void scan_keep_u32(const uint8_t* flags, uint64_t n, uint32_t* out, const ScanWs& ws, hipStream_t st);
void scan_u32(const uint32_t* in, uint64_t n, uint32_t* out, const ScanWs& ws, hipStream_t st);
void scan_len_u64(const uint32_t* ids, const uint64_t* offsets, uint64_t n, uint64_t* out, const ScanWs& ws,
                  hipStream_t st);
void scan_wrap_pieces_u32(const uint32_t* ids, const uint64_t* offsets, const uint64_t* opre,
                          const uint64_t* src_doc_start, const uint16_t* source, const uint64_t* start, uint32_t T,
                          uint64_t n, uint32_t* out, const ScanWs& ws, hipStream_t st);
void scan_pieces_u32(const uint32_t* ids, const uint64_t* offsets, const uint64_t* opre,
                     const uint64_t* src_doc_start, const uint16_t* source, const uint64_t* start, uint32_t T,
                     uint64_t n, uint32_t* out, const ScanWs& ws, hipStream_t st);

}  // namespace dp
