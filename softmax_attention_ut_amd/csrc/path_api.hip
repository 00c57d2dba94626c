// C ABI of libpath_attn.so: argument checks, workspace planning, launches.
// Declarations and contracts: include/path_attn.h.
#include "path_attn.h"
#include "path_internal.h"

using namespace path;

namespace {

constexpr int kBf16Chunk = 64;

bool valid_dtype(int dt) { return dt == PATH_F32 || dt == PATH_BF16; }

int default_chunk(int d, int dt) {
    if (dt == PATH_BF16) return kBf16Chunk;
    return d <= 32 ? 16 : 32;
}

// 0 = ok, else a path_status_t
int check_fwd_shape(int B, int H, int L, int d, int dt, int& chunk) {
    if (B < 1 || H < 1 || L < 1 || !valid_dtype(dt)) return PATH_ERR_INVALID;
    if ((long long)B * H * L > (1LL << 31) / 4) return PATH_ERR_UNSUPPORTED;
    if (chunk == 0) chunk = default_chunk(d, dt);
    if (dt == PATH_BF16) {
        if (d != 64 && d != 128) return PATH_ERR_UNSUPPORTED;
        if (chunk != kBf16Chunk) return PATH_ERR_UNSUPPORTED;
    } else {
        if (d != 16 && d != 32 && d != 64 && d != 128) return PATH_ERR_UNSUPPORTED;
        if (chunk != 16 && chunk != 32 && chunk != 64) return PATH_ERR_UNSUPPORTED;
        if (d == 128 && chunk > 32) return PATH_ERR_UNSUPPORTED;
    }
    return PATH_OK;
}

Workspace fwd_plan(int B, int H, int L, int d, int dt, int chunk, bool gate, bool with_z) {
    return plan_workspace((size_t)B * H, (size_t)L, (size_t)d, (size_t)chunk, dt == PATH_BF16,
                          gate, with_z);
}

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

}  // namespace

extern "C" {

const char* path_status_string(int status) {
    switch (status) {
        case PATH_OK: return "ok";
        case PATH_ERR_INVALID: return "invalid argument";
        case PATH_ERR_UNSUPPORTED: return "unsupported size or chunk";
        case PATH_ERR_HIP: return "HIP runtime or launch error";
        case PATH_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

const char* path_version(void) { return "path_attn 0.1 (gfx950)"; }

size_t path_attn_fwd_workspace_bytes(int B, int H, int L, int d, int dtype, int chunk) {
    if (check_fwd_shape(B, H, L, d, dtype, chunk) != PATH_OK) return 0;
    // the gate sections are always reserved so one size fits both variants
    return fwd_plan(B, H, L, d, dtype, chunk, true, false).total;
}

}  // extern "C"

namespace {

struct FwdPlan {
    Workspace ws;
    int BH, N;
    bool gate, bf;
};

int plan_fwd(int B, int H, int L, int d, int dtype, int& chunk, bool gate, const void* workspace,
             size_t ws_bytes, FwdPlan& p) {
    int st = check_fwd_shape(B, H, L, d, dtype, chunk);
    if (st != PATH_OK) return st;
    p.ws = fwd_plan(B, H, L, d, dtype, chunk, gate, false);
    if (!workspace || ws_bytes < p.ws.total) return PATH_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return PATH_ERR_WORKSPACE;
    p.BH = B * H;
    p.N = (L + chunk - 1) / chunk;
    p.gate = gate;
    p.bf = dtype == PATH_BF16;
    return PATH_OK;
}

// Sections at offset 0 other than kt (which always comes first) are absent.
UtArgs ut_args(const FwdPlan& p, const void* q, float scale, const void* k, const void* v,
               const void* w, const float* beta, const float* log_f, int L, int d, int chunk,
               void* workspace, bool with_z) {
    UtArgs u{};
    u.k = k; u.v = v; u.w = w; u.beta = beta; u.log_f = log_f;
    u.BH = p.BH; u.L = L; u.N = p.N; u.C = chunk; u.D = d;
    u.kt = at(workspace, p.ws.kt);
    u.ut = p.ws.ut ? at(workspace, p.ws.ut) : nullptr;
    u.vt = p.ws.vt ? at(workspace, p.ws.vt) : nullptr;
    u.yt = p.ws.yt ? at(workspace, p.ws.yt) : nullptr;
    u.zt = with_z ? at(workspace, p.ws.zt) : nullptr;
    u.q = p.ws.qt ? q : nullptr;
    u.scale2 = scale * kLog2e;
    u.qt = p.ws.qt ? at(workspace, p.ws.qt) : nullptr;
    u.pd = p.ws.pd ? at(workspace, p.ws.pd) : nullptr;
    u.ml = p.ws.ml ? reinterpret_cast<float*>(at(workspace, p.ws.ml)) : nullptr;
    u.mt = p.ws.mt ? at(workspace, p.ws.mt) : nullptr;
    u.loc = p.gate ? reinterpret_cast<float*>(at(workspace, p.ws.loc)) : nullptr;
    u.csum = p.gate ? reinterpret_cast<float*>(at(workspace, p.ws.csum)) : nullptr;
    u.gb = p.ws.gb ? at(workspace, p.ws.gb) : nullptr;
    return u;
}

}  // namespace

extern "C" {

int path_attn_fwd_prepare(const void* q, const void* k, const void* v, const void* w,
                          const float* beta, const float* log_f, int B, int H, int L, int d,
                          float scale, int dtype, int chunk, void* workspace, size_t ws_bytes,
                          void* stream) {
    FwdPlan p;
    int st = plan_fwd(B, H, L, d, dtype, chunk, log_f != nullptr, workspace, ws_bytes, p);
    if (st != PATH_OK) return st;
    if (!q || !k || !v || !w || !beta) return PATH_ERR_INVALID;
    if (!(scale == scale)) return PATH_ERR_INVALID;
    const UtArgs u = ut_args(p, q, scale, k, v, w, beta, log_f, L, d, chunk, workspace, false);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = p.bf ? launch_path_ut_bf16(u, s) : launch_path_ut_f32(u, s);
    return e == hipSuccess ? PATH_OK : PATH_ERR_HIP;
}

int path_attn_fwd_scan(const void* q, const void* k, const void* v, const void* w,
                       const float* log_f, void* out, float* lse, int B, int H, int L, int d,
                       float scale, int dtype, int chunk, const void* workspace, size_t ws_bytes,
                       void* stream) {
    FwdPlan p;
    void* wsp = const_cast<void*>(workspace);
    int st = plan_fwd(B, H, L, d, dtype, chunk, log_f != nullptr, wsp, ws_bytes, p);
    if (st != PATH_OK) return st;
    if (!q || !k || !v || !w || !out) return PATH_ERR_INVALID;
    if (!(scale == scale)) return PATH_ERR_INVALID;
    const UtArgs u = ut_args(p, q, scale, k, v, w, nullptr, log_f, L, d, chunk, wsp, false);
    FwdArgs f{};
    f.q = q; f.k = k; f.v = v; f.w = w;
    f.kt = u.kt; f.ut = u.ut; f.vt = u.vt; f.yt = u.yt; f.mt = u.mt;
    f.loc = u.loc; f.csum = u.csum; f.gb = u.gb;
    f.qt = u.qt; f.pd = u.pd; f.ml = u.ml;
    f.out = out; f.lse = lse;
    f.BH = p.BH; f.L = L; f.N = p.N; f.C = chunk; f.D = d;
    f.nqb = (p.N + 1) / 2;
    f.scale2 = scale * kLog2e;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = p.bf ? launch_path_fwd_bf16(f, p.gate, s) : launch_path_fwd_f32(f, p.gate, s);
    return e == hipSuccess ? PATH_OK : PATH_ERR_HIP;
}

int path_attn_fwd(const void* q, const void* k, const void* v, const void* w,
                  const float* beta, const float* log_f, void* out, float* lse,
                  int B, int H, int L, int d, float scale, int dtype, int chunk,
                  void* workspace, size_t ws_bytes, void* stream) {
    if (!q || !out) return PATH_ERR_INVALID;
    int st = path_attn_fwd_prepare(q, k, v, w, beta, log_f, B, H, L, d, scale, dtype, chunk,
                                   workspace, ws_bytes, stream);
    if (st != PATH_OK) return st;
    return path_attn_fwd_scan(q, k, v, w, log_f, out, lse, B, H, L, d, scale, dtype, chunk,
                              workspace, ws_bytes, stream);
}

size_t path_attn_bwd_workspace_bytes(int B, int H, int L, int d, int dtype) {
    int chunk = kBf16Chunk;
    if (dtype != PATH_BF16 || d != 64 || check_fwd_shape(B, H, L, d, dtype, chunk) != PATH_OK)
        return 0;
    return plan_bwd_workspace((size_t)B * H, (size_t)L).total;
}

int path_attn_bwd(const void* q, const void* k, const void* v, const void* w,
                  const float* beta, const float* log_f, const void* out, const float* lse,
                  const void* d_out, float* dq, float* dk, float* dv, float* dw, float* dbeta,
                  float* dlog_f, int B, int H, int L, int d, float scale, int dtype,
                  void* workspace, size_t ws_bytes, void* stream) {
    int chunk = kBf16Chunk;
    int st = check_fwd_shape(B, H, L, d, dtype, chunk);
    if (st != PATH_OK) return st;
    if (dtype != PATH_BF16 || d != 64) return PATH_ERR_UNSUPPORTED;
    if (!q || !k || !v || !w || !beta || !out || !lse || !d_out) return PATH_ERR_INVALID;
    if (!dq || !dk || !dv || !dw || !dbeta) return PATH_ERR_INVALID;
    if ((log_f == nullptr) != (dlog_f == nullptr)) return PATH_ERR_INVALID;
    if (!(scale == scale)) return PATH_ERR_INVALID;
    const BwdWorkspace ws = plan_bwd_workspace((size_t)B * H, (size_t)L);
    if (!workspace || ws_bytes < ws.total) return PATH_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return PATH_ERR_WORKSPACE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int BH = B * H, N = (L + chunk - 1) / chunk;
    // the forward's per-chunk quantities (K~, -U^T, Y^T, -M^T, gate sums)
    UtArgs u{};
    u.k = k; u.v = v; u.w = w; u.beta = beta; u.log_f = log_f;
    u.BH = BH; u.L = L; u.N = N; u.C = chunk; u.D = d;
    u.kt = at(workspace, ws.fwd.kt);
    u.ut = at(workspace, ws.fwd.ut);
    u.yt = at(workspace, ws.fwd.yt);
    u.mt = at(workspace, ws.fwd.mt);
    u.loc = log_f ? reinterpret_cast<float*>(at(workspace, ws.fwd.loc)) : nullptr;
    u.csum = log_f ? reinterpret_cast<float*>(at(workspace, ws.fwd.csum)) : nullptr;
    if (launch_path_ut_bf16(u, s) != hipSuccess) return PATH_ERR_HIP;
    BwdArgs b{};
    b.q = q; b.k = k; b.v = v; b.w = w; b.beta = beta; b.log_f = log_f;
    b.out = out; b.lse = lse; b.dout = d_out;
    b.dq = dq; b.dk = dk; b.dv = dv; b.dw = dw; b.dbeta = dbeta; b.dlogf = dlog_f;
    b.kt = u.kt; b.ut = u.ut; b.yt = u.yt; b.mt = u.mt; b.loc = u.loc; b.csum = u.csum;
    b.kp = at(workspace, ws.kp);
    b.kts = at(workspace, ws.kts);
    b.mn = at(workspace, ws.mn);
    b.mtn = at(workspace, ws.mtn);
    b.qs = at(workspace, ws.qs);
    b.gs = at(workspace, ws.gs);
    b.own = reinterpret_cast<float*>(at(workspace, ws.own));
    b.dsum = reinterpret_cast<float*>(at(workspace, ws.dsum));
    b.rsum = reinterpret_cast<float*>(at(workspace, ws.rsum));
    b.csd = reinterpret_cast<float*>(at(workspace, ws.csd));
    b.csl = reinterpret_cast<float*>(at(workspace, ws.csl));
    b.BH = BH; b.L = L; b.N = N; b.scale = scale;
    return launch_path_bwd(b, s) == hipSuccess ? PATH_OK : PATH_ERR_HIP;
}

size_t path_kcache_workspace_bytes(int B, int H, int L, int d, int dtype) {
    int chunk = kBf16Chunk;
    if (dtype != PATH_BF16 || check_fwd_shape(B, H, L, d, dtype, chunk) != PATH_OK) return 0;
    return fwd_plan(B, H, L, d, dtype, chunk, false, true).total;
}

}  // extern "C"

static int kcache_from_prefill(const void* k, const void* v, const void* w, const float* beta,
                               void* k_cache, void* v_cache, int B, int H, int L, int T_max,
                               int d, int dtype, void* workspace, size_t ws_bytes, void* stream,
                               const CacheMap& map) {
    int chunk = kBf16Chunk;
    if (!valid_dtype(dtype)) return PATH_ERR_INVALID;
    if (dtype != PATH_BF16) return PATH_ERR_UNSUPPORTED;
    int st = check_fwd_shape(B, H, L, d, dtype, chunk);
    if (st != PATH_OK) return st;
    if (T_max < L) return PATH_ERR_INVALID;
    if (!k || !v || !w || !beta || !k_cache || !v_cache) return PATH_ERR_INVALID;
    const Workspace ws = fwd_plan(B, H, L, d, dtype, chunk, false, true);
    if (!workspace || ws_bytes < ws.total) return PATH_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return PATH_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int BH = B * H, N = (L + chunk - 1) / chunk;
    UtArgs u{};
    u.k = k; u.v = v; u.w = w; u.beta = beta; u.log_f = nullptr;
    u.BH = BH; u.L = L; u.N = N; u.C = chunk; u.D = d;
    u.kt = at(workspace, ws.kt);
    u.zt = at(workspace, ws.zt);            // the hand-off needs K~ and Z only
    if (launch_path_ut_bf16(u, s) != hipSuccess) return PATH_ERR_HIP;
    KcacheArgs c{};
    c.kt = u.kt; c.kt_in = u.kt; c.w = w; c.zt = u.zt; c.v = v;
    c.k_cache = k_cache; c.v_cache = v_cache;
    c.BH = BH; c.L = L; c.N = N; c.T_max = T_max;
    c.NG = (N + kKcacheGroup - 1) / kKcacheGroup;
    c.tg = reinterpret_cast<float*>(at(workspace, ws.tg));
    c.rg = at(workspace, ws.rg);
    c.map = map;
    return launch_path_kcache(c, d, s) == hipSuccess ? PATH_OK : PATH_ERR_HIP;
}

static int kcache_from_forward(const void* fwd_workspace, size_t fwd_ws_bytes, const void* v,
                               void* k_cache, void* v_cache, int B, int H, int L, int T_max,
                               int d, int dtype, void* workspace, size_t ws_bytes, void* stream,
                               const CacheMap& map) {
    int chunk = kBf16Chunk;
    if (!valid_dtype(dtype)) return PATH_ERR_INVALID;
    if (dtype != PATH_BF16) return PATH_ERR_UNSUPPORTED;
    int st = check_fwd_shape(B, H, L, d, dtype, chunk);
    if (st != PATH_OK) return st;
    if (T_max < L) return PATH_ERR_INVALID;
    if (!v || !k_cache || !v_cache) return PATH_ERR_INVALID;
    // the forward's workspace: K~ and -M^T sit before the sections that the
    // gate adds, so their offsets do not depend on it
    const Workspace fw = fwd_plan(B, H, L, d, dtype, chunk, false, false);
    const size_t fw_need = fwd_plan(B, H, L, d, dtype, chunk, true, false).total;   // path_attn_fwd_workspace_bytes
    if (!fwd_workspace || !fw.mt || fwd_ws_bytes < fw_need) return PATH_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(fwd_workspace) & 255) return PATH_ERR_WORKSPACE;
    const Workspace ws = fwd_plan(B, H, L, d, dtype, chunk, false, true);
    if (!workspace || ws_bytes < ws.total) return PATH_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return PATH_ERR_WORKSPACE;
    const int BH = B * H, N = (L + chunk - 1) / chunk;
    void* fwsp = const_cast<void*>(fwd_workspace);
    KcacheArgs c{};
    c.kt = at(workspace, ws.kt);
    c.kt_in = at(fwsp, fw.kt);
    c.mt = at(fwsp, fw.mt);
    c.v = v;
    c.k_cache = k_cache; c.v_cache = v_cache;
    c.BH = BH; c.L = L; c.N = N; c.T_max = T_max;
    c.NG = (N + kKcacheGroup - 1) / kKcacheGroup;
    c.tg = reinterpret_cast<float*>(at(workspace, ws.tg));
    c.rg = at(workspace, ws.rg);
    c.map = map;
    return launch_path_kcache(c, d, static_cast<hipStream_t>(stream)) == hipSuccess ? PATH_OK : PATH_ERR_HIP;
}

// 0 = ok: a page pool of num_blocks pages of `page` slots (a multiple of
// 64), each sequence's pages listed in block_table [B][max_blocks]
static int check_pages(const int* block_table, int num_blocks, int max_blocks, int page,
                       int H, CacheMap& map) {
    if (!block_table || num_blocks < 1 || max_blocks < 1 || page < 1) return PATH_ERR_INVALID;
    if (page % 64 != 0) return PATH_ERR_UNSUPPORTED;
    if ((long long)max_blocks * page >= (1LL << 31)) return PATH_ERR_UNSUPPORTED;
    if ((long long)num_blocks * H * page >= (1LL << 40)) return PATH_ERR_UNSUPPORTED;
    map = CacheMap{block_table, page, max_blocks, num_blocks, H, max_blocks * page};
    return PATH_OK;
}

extern "C" {

int path_kcache_from_prefill(const void* k, const void* v, const void* w, const float* beta,
                             void* k_cache, void* v_cache, int B, int H, int L, int T_max,
                             int d, int dtype, void* workspace, size_t ws_bytes, void* stream) {
    const CacheMap map{nullptr, 0, 0, 0, H, T_max};
    return kcache_from_prefill(k, v, w, beta, k_cache, v_cache, B, H, L, T_max, d, dtype,
                               workspace, ws_bytes, stream, map);
}

int path_kcache_from_forward(const void* fwd_workspace, size_t fwd_ws_bytes, const void* v,
                             void* k_cache, void* v_cache, int B, int H, int L, int T_max,
                             int d, int dtype, void* workspace, size_t ws_bytes, void* stream) {
    const CacheMap map{nullptr, 0, 0, 0, H, T_max};
    return kcache_from_forward(fwd_workspace, fwd_ws_bytes, v, k_cache, v_cache, B, H, L, T_max,
                               d, dtype, workspace, ws_bytes, stream, map);
}

int path_kcache_from_prefill_paged(const void* k, const void* v, const void* w,
                                   const float* beta, void* k_pool, void* v_pool,
                                   const int* block_table, int num_blocks, int max_blocks,
                                   int page, int B, int H, int L, int d, int dtype,
                                   void* workspace, size_t ws_bytes, void* stream) {
    CacheMap map{};
    const int st = check_pages(block_table, num_blocks, max_blocks, page, H, map);
    if (st != PATH_OK) return st;
    return kcache_from_prefill(k, v, w, beta, k_pool, v_pool, B, H, L, map.T_max, d, dtype,
                               workspace, ws_bytes, stream, map);
}

size_t path_decode_workspace_bytes(int B, int H, int T_max, int d, int dtype) {
    if (B < 1 || H < 1 || T_max < 1 || dtype != PATH_BF16 || (d != 64 && d != 128)) return 0;
    const size_t nsplit_max = ((size_t)T_max + kDecodeSplitQuantum - 1) / kDecodeSplitQuantum;
    return align256((size_t)B * H * nsplit_max * (d + 2) * sizeof(float));
}

static int decode_check(void* k_cache, void* v_cache, const void* q_t, const void* k_t,
                        const void* v_t, const void* w_t, const float* beta_t, void* out_t,
                        int B, int H, int t, int T_max, int d, float scale, int dtype) {
    if (B < 1 || H < 1 || T_max < 1 || t < 0 || t >= T_max || !valid_dtype(dtype))
        return PATH_ERR_INVALID;
    if (dtype != PATH_BF16 || (d != 64 && d != 128)) return PATH_ERR_UNSUPPORTED;
    if (!k_cache || !v_cache || !q_t || !k_t || !v_t || !w_t || !beta_t || !out_t)
        return PATH_ERR_INVALID;
    if (!(scale == scale)) return PATH_ERR_INVALID;
    return PATH_OK;
}

// The step itself, after the checks; part holds the split partials.
static int decode_launch(void* k_cache, void* v_cache, float* f_cache, const void* q_t,
                         const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                         const float* log_f_t, void* out_t, float* lse_t, int B, int H, int t,
                         int T_max, int d, float scale, void* part, void* stream,
                         const CacheMap& map) {
    DecodeArgs a{};
    a.k_cache = k_cache; a.v_cache = v_cache;
    a.q = q_t; a.k = k_t; a.v = v_t; a.w = w_t; a.beta = beta_t;
    a.out = out_t; a.lse = lse_t;
    a.part = static_cast<float*>(part);
    a.BH = B * H; a.t = t; a.T_max = T_max;
    a.scale2 = scale * kLog2e;
    a.log_f = log_f_t; a.f_cache = f_cache;
    a.map = map;
    return launch_path_decode(a, d, static_cast<hipStream_t>(stream)) == hipSuccess
               ? PATH_OK : PATH_ERR_HIP;
}

static int decode_step(void* k_cache, void* v_cache, float* f_cache, const void* q_t,
                       const void* k_t, const void* v_t, const void* w_t, const float* beta_t,
                       const float* log_f_t, void* out_t, float* lse_t, int B, int H, int t,
                       int T_max, int d, float scale, int dtype, void* workspace, size_t ws_bytes,
                       void* stream, const CacheMap& map) {
    const int st = decode_check(k_cache, v_cache, q_t, k_t, v_t, w_t, beta_t, out_t, B, H, t,
                                T_max, d, scale, dtype);
    if (st != PATH_OK) return st;
    const size_t need = path_decode_workspace_bytes(B, H, T_max, d, dtype);
    if (!workspace || ws_bytes < need) return PATH_ERR_WORKSPACE;
    return decode_launch(k_cache, v_cache, f_cache, q_t, k_t, v_t, w_t, beta_t, log_f_t, out_t,
                         lse_t, B, H, t, T_max, d, scale, workspace, stream, map);
}

int path_decode_step(void* k_cache, void* v_cache, const void* q_t, const void* k_t,
                     const void* v_t, const void* w_t, const float* beta_t, void* out_t,
                     float* lse_t, int B, int H, int t, int T_max, int d, float scale,
                     int dtype, void* workspace, size_t ws_bytes, void* stream) {
    const CacheMap map{nullptr, 0, 0, 0, H, T_max};
    return decode_step(k_cache, v_cache, nullptr, q_t, k_t, v_t, w_t, beta_t, nullptr, out_t, lse_t,
                       B, H, t, T_max, d, scale, dtype, workspace, ws_bytes, stream, map);
}

int path_decode_step_noalloc(void* k_cache, void* v_cache, const void* q_t, const void* k_t,
                             const void* v_t, const void* w_t, const float* beta_t, void* out_t,
                             float* lse_t, int B, int H, int t, int T_max, int d, float scale,
                             int dtype, void* stream) {
    const int st = decode_check(k_cache, v_cache, q_t, k_t, v_t, w_t, beta_t, out_t, B, H, t,
                                T_max, d, scale, dtype);
    if (st != PATH_OK) return st;
    // the step uses at most ceil((t + 1) / 64) splits per head
    const size_t nsplit_max = ((size_t)t + kDecodeSplitQuantum) / kDecodeSplitQuantum;
    if ((size_t)B * H * nsplit_max * (d + 2) * sizeof(float) > kDecodeScratchBytes)
        return PATH_ERR_WORKSPACE;
    void* part = nullptr;
    if (decode_scratch(&part) != hipSuccess) return PATH_ERR_HIP;
    const CacheMap map{nullptr, 0, 0, 0, H, T_max};
    return decode_launch(k_cache, v_cache, nullptr, q_t, k_t, v_t, w_t, beta_t, nullptr, out_t,
                         lse_t, B, H, t, T_max, d, scale, part, stream, map);
}

int path_fcache_from_prefill(const float* log_f, float* f_cache, int B, int H, int L, int T_max,
                             void* stream) {
    if (B < 1 || H < 1 || L < 1 || T_max < L || !log_f || !f_cache) return PATH_ERR_INVALID;
    FcacheArgs a{};
    a.log_f = log_f; a.f_cache = f_cache;
    a.BH = B * H; a.L = L; a.T_max = T_max;
    return launch_path_fcache(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PATH_OK
                                                                                 : PATH_ERR_HIP;
}

int path_decode_step_gated(void* k_cache, void* v_cache, float* f_cache, const void* q_t,
                           const void* k_t, const void* v_t, const void* w_t,
                           const float* beta_t, const float* log_f_t, void* out_t, float* lse_t,
                           int B, int H, int t, int T_max, int d, float scale, int dtype,
                           void* workspace, size_t ws_bytes, void* stream) {
    if (!f_cache || !log_f_t) return PATH_ERR_INVALID;
    const CacheMap map{nullptr, 0, 0, 0, H, T_max};
    return decode_step(k_cache, v_cache, f_cache, q_t, k_t, v_t, w_t, beta_t, log_f_t, out_t,
                       lse_t, B, H, t, T_max, d, scale, dtype, workspace, ws_bytes, stream, map);
}

int path_decode_step_paged(void* k_pool, void* v_pool, const int* block_table, int num_blocks,
                           int max_blocks, int page, float* f_cache, const float* log_f_t,
                           const void* q_t, const void* k_t, const void* v_t, const void* w_t,
                           const float* beta_t, void* out_t, float* lse_t, int B, int H, int t,
                           int d, float scale, int dtype, void* workspace, size_t ws_bytes,
                           void* stream) {
    if ((f_cache == nullptr) != (log_f_t == nullptr)) return PATH_ERR_INVALID;
    if (B < 1 || H < 1) return PATH_ERR_INVALID;
    CacheMap map{};
    const int st = check_pages(block_table, num_blocks, max_blocks, page, H, map);
    if (st != PATH_OK) return st;
    return decode_step(k_pool, v_pool, f_cache, q_t, k_t, v_t, w_t, beta_t, log_f_t, out_t,
                       lse_t, B, H, t, map.T_max, d, scale, dtype, workspace, ws_bytes, stream,
                       map);
}

}  // extern "C"
