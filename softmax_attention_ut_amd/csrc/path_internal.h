// Internal declarations shared by the PaTH HIP kernels and the C-ABI layer.
// gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace path {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Operand-slot permutation.
//
// In the 32x32x16 bf16 MFMA the fp32 accumulator of a 32x32 tile gives lane l
// the rows 8*(v/4) + 4*(l/32) + (v%4), v = 0..15, of column l%32.  The
// B operand of the same instruction wants lane l to hold 8 consecutive
// k-slots 8*(l/32)..+7 of column l%32.  Handing accumulator registers
// v = 8*s .. 8*s+7 straight to the next MFMA as the B operand of k-step s
// therefore assigns k-slot 16*s + p to row 16*s + perm16(p), where perm16
// swaps the middle two groups of four: 0-3, 8-11, 4-7, 12-15.  Every operand
// that meets such a chained accumulator along k is stored with its k axis
// permuted the same way, so no register shuffles are needed between the
// chained products.  perm16 is an involution.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int perm16(int p) {
    return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
}
__host__ __device__ constexpr int permk(int s) {  // applied inside each group of 16
    return (s & ~15) | perm16(s & 15);
}

// ---------------------------------------------------------------------------
// Workspace layout of the forward pass (byte offsets, 256-aligned sections).
// N = number of chunks, Lp = N * C.
//   bf16 mode (C = 64):
//     kt  [BH][Lp][D]   bf16  keys carried to their chunk end (natural rows)
//     ut  [BH][N][D][C] bf16  -U^T (U = T^{-1} W): [rho][sigma] = -U[permk(sigma)][permk(rho)]
//     vt  [BH][N][D][C] bf16  V^T, laid out like ut (d = 128; the d = 64 scan
//                             reads V as it is with LDS transpose loads)
//     yt  [BH][N][C][C] bf16  Y^T (Y = T^{-1} strictLower(W K^T)): [j][sigma] = Y[permk(sigma)][j]
//     zt  [BH][N][D][C] bf16  -Z^T (Z = T^{-T} W), laid out like ut (cache only)
//     mt  [BH][N][D][D] bf16  -M^T, M = W^T U: [rho][d'] = -M[d'][permk(rho)]
//                             (forward: dense d x d transport)
//   The bf16 forward has no ut / yt: its prepare stage also takes each
//   query chunk's own-chunk (diagonal) step and writes instead
//     qt  [BH][Lp][D]  bf16  the query carried to its chunk start,
//                            q - lower(q W^T) U, times scale*log2(e)
//     pd  [BH][Lp][C]  bf16  the query's own-chunk probabilities
//                            exp2(z_ij - m_i), in the scan's B-operand
//                            register order (see path_ut_bf16.hip)
//     ml  [BH][Lp][2]  f32   (m_i, l_i): their maximum (log2 units) and sum
//   Permuting the d rows of the transposed tiles makes the fp32 accumulators
//   they multiply into (carried query, output) come out with register 8s+t
//   holding d = 16s + 8*(lane/32) + t, i.e. in natural B-operand order.
//   f32 mode:
//     kt  [BH][Lp][D] f32, u [BH][Lp][D] f32, y [BH][N][C][C] f32 (natural)
//   both (forget gate only):
//     loc  [BH][Lp] f32  -sum_{s=j+1}^{chunk end} log2 f_s
//     csum [BH][N]  f32  sum over the chunk of log2 f_s
// ---------------------------------------------------------------------------
// Chunks per group of the key-cache hand-off's suffix products.
constexpr int kKcacheGroup = 8;

struct Workspace {
    size_t kt, ut, vt, yt, zt, mt, loc, csum, gb, qt, pd, ml, tg, rg, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The bf16 forward carries queries through whole chunks with the d x d
// product (2 d^2 flops per query and chunk, against 4 C d for the rank-C
// form: half at d = 64, the same at d = 128 = 2C, where it needs one operand
// tile per chunk instead of two and no intermediate Q W^T).
inline bool dense_transport(size_t D, bool bf16_mode) { return bf16_mode && (D == 64 || D == 128); }

inline Workspace plan_workspace(size_t BH, size_t L, size_t D, size_t C,
                                bool bf16_mode, bool gate, bool with_z) {
    Workspace w{};
    const size_t N = (L + C - 1) / C, Lp = N * C;
    const size_t es = bf16_mode ? 2 : 4;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    // the bf16 forward: own-chunk step in the prepare stage (no ut / yt)
    // the key-cache hand-off (with_z): kt, zt and the group products only
    const bool diag = !with_z && dense_transport(D, bf16_mode);
    const size_t NG = (N + kKcacheGroup - 1) / kKcacheGroup;
    w.kt = take(BH * Lp * D * es);
    w.ut = (diag || with_z) ? 0 : take(BH * Lp * D * es);
    w.vt = (bf16_mode && D != 64 && !with_z) ? take(BH * Lp * D * es) : 0;
    w.yt = (diag || with_z) ? 0 : take(BH * N * C * C * es);
    w.zt = with_z ? take(BH * Lp * D * es) : 0;
    w.tg = with_z ? take(BH * NG * D * D * 4) : 0;
    w.rg = with_z ? take(BH * NG * 2 * D * D * 2) : 0;
    w.mt = diag ? take(BH * N * D * D * es) : 0;
    w.qt = diag ? take(BH * Lp * D * es) : 0;
    w.pd = diag ? take(BH * Lp * C * es) : 0;
    w.ml = diag ? take(BH * Lp * 2 * 4) : 0;
    w.loc = gate ? take(BH * Lp * 4) : 0;
    w.csum = gate ? take(BH * N * 4) : 0;
    // d x d transport with the gate: each key's gate term as the A row of the
    // logit product's bias k-step, 16 bf16 per key
    w.gb = (gate && w.mt) ? take(BH * Lp * 16 * es) : 0;
    w.total = off;
    return w;
}

// ---------------------------------------------------------------------------
// Kernel argument blocks.
// ---------------------------------------------------------------------------
struct UtArgs {
    const void* q;         // bf16 forward: queries of the own-chunk step (else null)
    float scale2;          // scale * log2(e) (own-chunk step)
    const void* k;
    const void* v;
    const void* w;
    const float* beta;
    const float* log_f;    // may be null
    int BH, L, N, C, D;
    void* kt;              // outputs (see Workspace)
    void* ut;
    void* vt;              // bf16 mode, d = 128 only (may be null)
    void* yt;
    void* zt;              // may be null
    void* mt;              // may be null (dense d x d transport tiles)
    float* loc;            // null without gate
    float* csum;
    void* gb;              // may be null (gate bias rows, d x d transport)
    void* qt;              // bf16 forward: own-chunk step outputs (else null)
    void* pd;
    float* ml;
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;         // w (and v in f32 mode) are read from the inputs
    const void* w;
    const void* kt;
    const void* ut;
    const void* vt;        // bf16 d = 128: V^T tiles (otherwise v is read)
    const void* yt;
    const void* mt;        // bf16: -M^T tiles
    const float* loc;
    const float* csum;
    const void* gb;        // bf16 with gate: bias rows of the key chunks
    const void* qt;        // bf16: own-chunk step results of the prepare stage
    const void* pd;
    const float* ml;
    void* out;
    float* lse;
    int BH, L, N, C, D, nqb;
    float scale2;          // scale * log2(e)
    int single;            // d = 64 scan: one query block per workgroup (set by the launcher)
};

// Where cache slot j of head bh = b * H + h lives, in rows of D elements:
// contiguous caches [BH][T_max][D] when `table` is null, else a page pool
// [num_blocks][H][page][D] with page `table[b * max_blocks + j / page]`.
// Pages outside [0, num_blocks) are never dereferenced (row < 0).
struct CacheMap {
    const int* table;      // [B][max_blocks] or null
    int page, max_blocks, num_blocks, H, T_max;
};

__device__ __forceinline__ long long cache_row(const CacheMap& c, int bh, int j) {
    if (!c.table) return (long long)bh * c.T_max + j;
    const int b = bh / c.H, h = bh - b * c.H;
    const int blk = c.table[(size_t)b * c.max_blocks + j / c.page];
    if (blk < 0 || blk >= c.num_blocks) return -1;
    return ((long long)blk * c.H + h) * c.page + (j % c.page);
}

struct KcacheArgs {
    void* kt;              // keys carried to their group's end (bf16), Y
    const void* kt_in;     // keys carried to their chunk end, K~ (the same buffer as kt, or the forward's)
    const void* w;         // input w [BH][L][D] (rank-C form)
    const void* zt;        // -Z^T tiles (rank-C form)
    const void* mt;        // the forward's -M^T tiles [BH][N][D][D] (dense form), else null
    const void* v;         // input values [BH][L][D]
    void* k_cache;         // contiguous [BH][T_max][D] or a page pool (see map)
    void* v_cache;
    int BH, L, N, T_max, NG;   // NG = ceil(N / kKcacheGroup)
    float* tg;             // [BH][NG][D][D] fp32: each group's product of chunk transforms
    void* rg;              // [BH][NG][2][D][D] bf16: suffix products, rows permuted, hi and lo
    CacheMap map;
};

struct DecodeArgs {
    void* k_cache;
    void* v_cache;
    const void* q;
    const void* k;
    const void* v;
    const void* w;
    const float* beta;
    void* out;
    float* lse;
    float* part;           // [BH][nsplit][D + 2] partial (o, m, l)
    int BH, t, T_max, nsplit, keys_per_split;   // split sizes: set by launch_path_decode
    float scale2;
    const float* log_f;    // [BH] log f_t, or null (no forget gate)
    float* f_cache;        // [BH][T_max] prefix sums of log f, or null (no forget gate)
    CacheMap map;          // K/V slot addresses (contiguous or paged)
};

struct FcacheArgs {
    const float* log_f;    // [BH][L]
    float* f_cache;        // [BH][T_max]
    int BH, L, T_max;
};

struct TransArgs {
    const void* x;         // [B][L][Dm] bf16
    const void* w_down;    // [R][Dm] bf16
    const void* w_up;      // [H*D][R] bf16
    const float* conv;     // [H*D][3]
    const void* u;         // [H][Dm] bf16
    const float* b;        // [H]
    void* w;               // [B][H][L][D] bf16
    float* beta;           // [B][H][L]
    int B, L, Dm, R, H, D, ntile;   // ntile: token tiles per sequence (set by the launcher)
};

// Decode splits are multiples of this many keys, so a head has at most
// ceil(T_max / kDecodeSplitQuantum) splits (the workspace holds that many).
constexpr int kDecodeSplitQuantum = 64;

// Backward pass (bf16, d = 64): inputs, outputs and its workspace sections
// (see path_bwd.hip).
struct BwdArgs {
    const void* q; const void* k; const void* v; const void* w;
    const float* beta; const float* log_f;   // log_f null without the gate
    const void* out; const float* lse; const void* dout;
    float* dq; float* dk; float* dv; float* dw; float* dbeta; float* dlogf;
    const void* kt; void* ut; void* yt; const void* mt;   // U, Y: made row-major in place
    void* kp; void* kts; void* mn; void* mtn;             // the chains' operand tiles
    const float* loc; const float* csum;
    void* qs; void* gs; float* own; float* dsum; float* rsum; float* csd; float* csl;
    int BH, L, N;
    float scale;
};

struct BwdWorkspace {
    Workspace fwd;         // kt, ut, yt, mt, loc, csum of the forward's prepare stage
    size_t kp, kts, mn, mtn, qs, gs, own, dsum, rsum, csd, csl, total;
};

inline BwdWorkspace plan_bwd_workspace(size_t BH, size_t L) {
    constexpr size_t C = 64, D = 64;
    BwdWorkspace b{};
    const size_t N = (L + C - 1) / C, Lp = N * C, pairs = N * (N - 1) / 2;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    b.fwd.kt = take(BH * Lp * D * 2);
    b.fwd.ut = take(BH * Lp * D * 2);
    b.fwd.yt = take(BH * N * C * C * 2);
    b.fwd.mt = take(BH * N * D * D * 2);
    b.fwd.loc = take(BH * Lp * 4);
    b.fwd.csum = take(BH * N * 4);
    b.kp = take(BH * N * C * D * 2);
    b.kts = take(BH * N * C * D * 2);
    b.mn = take(BH * N * D * D * 2);
    b.mtn = take(BH * N * D * D * 2);
    b.qs = take(BH * pairs * C * D * 2);
    b.gs = take(BH * pairs * C * D * 2);
    b.own = take(BH * N * 11 * C * D * 4);
    b.dsum = take(BH * Lp * 4);
    b.rsum = take(BH * Lp * 4);
    b.csd = take(BH * Lp * 4);
    b.csl = take(BH * Lp * 4);
    b.total = off;
    return b;
}

// Host-side launchers (return hipError_t of the launch).
hipError_t launch_path_ut_f32(const UtArgs& a, hipStream_t s);
hipError_t launch_path_ut_bf16(const UtArgs& a, hipStream_t s);
hipError_t launch_path_fwd_f32(const FwdArgs& a, bool gate, hipStream_t s);
hipError_t launch_path_fwd_bf16(const FwdArgs& a, bool gate, hipStream_t s);
hipError_t launch_path_kcache(const KcacheArgs& a, int D, hipStream_t s);
hipError_t launch_path_decode(const DecodeArgs& a, int D, hipStream_t s);
hipError_t launch_path_bwd(const BwdArgs& a, hipStream_t s);
// The library's own split-partials buffer of path_decode_step_noalloc: its
// size, and its device address on the current device (looked up once per
// device with hipGetSymbolAddress, then cached).
constexpr size_t kDecodeScratchBytes = size_t(8) << 20;
hipError_t decode_scratch(void** ptr);
hipError_t launch_path_fcache(const FcacheArgs& a, hipStream_t s);
hipError_t launch_path_transition(TransArgs a, hipStream_t s);

// ---------------------------------------------------------------------------
// A operands of a 32x32x16 bf16 MFMA that are the transpose of a tile kept
// as it is: a [rows][64] bf16 tile T in LDS (rows of 128 bytes, 16-byte units
// swizzled by swz_v) gives A[r][s] = T[permk(s)][permk(r)] for output row r
// (32 dt + lane % 32) and k-slot s of k-step ks.  The d = 64 scan takes its
// PV operand V^T this way from the V tile ([token][d]), and the key-cache
// hand-off its -M operand from the -M^T tiles of the forward's workspace.
//
// Within each group of 16 lanes, ds_read_b64_tr_b16 gives lane i, element t,
// the element i % 4 of the 8 bytes read by lane 4t + i/4.  So lane 4t + q
// reads 4 consecutive columns of one row, and every lane receives one column
// of four rows.  The permutations of the row (k-slot) and column (output row)
// axes act on blocks of four, which this access respects.  The operand of
// k-step ks, rows dt, takes two loads (slots 0-3 and 4-7); a lane's 8 byte
// offsets depend on (ks & 1, load, dt), the rows 32 (ks >> 1) further on add
// 4096 bytes.
//
// One transpose load reads 8 bytes per lane: lanes 0-31 cover 64 bytes of each
// of 4 consecutive rows, lanes 32-63 the next 4 rows (two 256-byte halves; by
// quarters, 16 lanes cover 32 bytes of each of 4 rows).  The swizzle gv(r)
// takes row bits 2, 0, 1 as unit bits 0, 1, 2: rows r and r + 2 then differ
// in unit bit 2, so the four rows' pieces of either half, or of any quarter,
// fall on distinct LDS banks (64 banks of 4 bytes for a 32-lane half, 32 for
// a 16-lane quarter).  The swizzle made for 16-byte row reads would put rows
// r and r + 2 on the same banks here.
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
__device__ __forceinline__ int swz_v(int r) {
    return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2);
}
__device__ __forceinline__ void vtr_offsets(unsigned off[8], int lane) {
    const int hh = lane >> 5, hp = (lane >> 4) & 1, j = lane & 15;
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
        for (int ins = 0; ins < 2; ++ins)
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                const int tok = permk(16 * par + 8 * hh + 4 * ins + (j >> 2));
                const int d = permk(32 * dt + 16 * hp + 4 * (j & 3));
                off[(par * 2 + ins) * 2 + dt] =
                    static_cast<unsigned>((tok * 64 + (((d >> 3) ^ swz_v(tok)) << 3) + (d & 7)) * 2);
            }
}
__device__ __forceinline__ bf16x8 pv_operand(const bf16* sv, const unsigned off[8], int dt, int ks) {
    const char* base = reinterpret_cast<const char*>(sv) + 4096 * (ks >> 1);
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + off[((ks & 1) * 2 + 0) * 2 + dt]));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + off[((ks & 1) * 2 + 1) * 2 + dt]));
    const v4s both[2] = {lo, hi};
    bf16x8 r;
    __builtin_memcpy(&r, both, sizeof(r));
    return r;
}

}  // namespace path
