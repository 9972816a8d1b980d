// C-ABI of the fused GEMM + ReLU: argument checks, configuration choice, launch.
//
// Semantics (page "TileLang：GPU/NPU 通用算子 DSL", §3.2 and §3.3): C is
// overwritten with max(A·op(B), 0); the grid has one workgroup per output tile
// and a ceil-divided K loop, so every shape is covered, tails included.
// gemm_relu_mx: the block-scaled (OCP MX) form of the same product (§4.1's
// MXFP8 / MXFP4).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "configs.hpp"
#include "gemm_relu.h"
#include "gemm_sp_relu_kernel.hpp"

using namespace gemm_relu_hip;

namespace gemm_relu_hip {
typedef hipError_t (*SpLaunchFn)(const SpArgs& args, int grid, hipStream_t stream);
SpLaunchFn launcher_sp(int in_dt, int out_dt, int transB, int variant);   // inst_sp.hip
}

namespace {

constexpr int kMaxDevices = 64;
constexpr int kNumCUs = 256;   // MI355X: 8 XCDs x 32 CUs

struct Env {
    bool sync = false;
    int force_cfg = -1;   // GEMM_RELU_FORCE_CONFIG=<name>
    int panel = 0;        // GEMM_RELU_PANEL=<tile rows>, 0 = default
    int nxcd = 8;         // GEMM_RELU_XCDS=<n>: 1 disables the XCD-aware tile remap
    int sk_units = 0;     // GEMM_RELU_SK_UNITS=<n>: stream-K units, 0 = one per CU
    int split_cols = -1;  // GEMM_RELU_SPLIT_COLS=<c>: two-region grid with c 256-wide tile
                          // columns first (0: never split); -1 = plan selection decides
    int pgrid = 0;        // GEMM_RELU_PERSISTENT_GRID=<n>: workgroups of a persistent
                          // configuration (0 = one per CU, at most one per tile)
    int splitk_parts = 0; // GEMM_RELU_SPLITK_PARTS=<n>: K parts of a K-split plan
                          // (0 = plan selection decides)
};

// Debug and tuning switches, read on every call so a process can change them
// between calls.
Env env()
{
    Env e;
    const char* s = std::getenv("GEMM_RELU_SYNC");
    e.sync = s && s[0] == '1';
    const char* f = std::getenv("GEMM_RELU_FORCE_CONFIG");
    if (f && f[0]) {
        for (int i = 0; i < CFG_COUNT; ++i)
            if (std::strcmp(f, config_info(i).name) == 0) e.force_cfg = i;
    }
    const char* p = std::getenv("GEMM_RELU_PANEL");
    if (p && p[0]) e.panel = std::atoi(p);
    const char* x = std::getenv("GEMM_RELU_XCDS");
    if (x && x[0]) e.nxcd = std::atoi(x) > 0 ? std::atoi(x) : 1;
    const char* u = std::getenv("GEMM_RELU_SK_UNITS");
    if (u && u[0]) e.sk_units = std::max(0, std::atoi(u));
    const char* c = std::getenv("GEMM_RELU_SPLIT_COLS");
    if (c && c[0]) e.split_cols = std::max(0, std::atoi(c));
    const char* pg = std::getenv("GEMM_RELU_PERSISTENT_GRID");
    if (pg && pg[0]) e.pgrid = std::max(0, std::atoi(pg));
    const char* sp = std::getenv("GEMM_RELU_SPLITK_PARTS");
    if (sp && sp[0]) e.splitk_parts = std::max(0, std::atoi(sp));
    return e;
}

// Per-device "is this a gfx950" cache.
struct DevState {
    std::once_flag once;
    bool ok = false;
    hipError_t err = hipSuccess;
};
DevState g_dev[kMaxDevices];

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_RELU_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return GEMM_RELU_EUNSUPPORTED;
    DevState& d = g_dev[dev];
    std::call_once(d.once, [&] {
        hipDeviceProp_t prop;
        d.err = hipGetDeviceProperties(&prop, dev);
        if (d.err == hipSuccess) d.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    });
    if (d.err != hipSuccess) return GEMM_RELU_EHIP;
    return d.ok ? GEMM_RELU_OK : GEMM_RELU_EUNSUPPORTED;
}

int elem_bytes(int dt)
{
    return dt == GEMM_RELU_F32 ? 4 : (dt == GEMM_RELU_F8_E4M3 || dt == GEMM_RELU_F8_E5M2) ? 1 : 2;
}

bool fp8_input(int dt) { return dt == GEMM_RELU_F8_E4M3 || dt == GEMM_RELU_F8_E5M2; }

bool overlaps(uintptr_t a, uint64_t na, uintptr_t b, uint64_t nb)
{
    if (na == 0 || nb == 0) return false;
    return a < b + nb && b < a + na;
}

struct Plan {
    int status = GEMM_RELU_OK;
    bool empty = false;   // nothing to launch
    int cfg = -1;
    int tiles_m = 0, tiles_n = 0;
    int dp_tiles = 0, sk_units = 0;   // stream-K configurations
    // two-region grid: cfg tiles over the first split columns, then cfg2
    // (d256x192x32_s4_i16) tiles over the rest
    int cfg2 = -1;
    int tiles1 = 0, tiles_m2 = 0, tiles_n2 = 0, n_org2 = 0;
    // K-split plan: `splits` parts of split_steps K steps per tile, ws_need
    // bytes of workspace
    int splits = 0, split_steps = 0;
    uint64_t ws_need = 0;
};



// ---- stream-K split (the 256x256 interleaved tile, selected by name only):
// whole rounds of tiles over the CUs keep one workgroup per tile; the
// remaining tiles' K steps go to `units` workgroups, one per CU unless
// GEMM_RELU_SK_UNITS sets the count.  Measured on MI355X it loses to one
// workgroup per tile on every shape tried (the fp32 partials and the
// cross-XCD cache write-back and invalidation cost more than the partly empty
// last round), so plan selection never chooses it.
constexpr int kSkMaxUnits = kNumCUs;    // the workspace holds 2 partials per unit

struct SkSplit {
    int dp_tiles = 0, units = 0;
};

SkSplit sk_split(int64_t tiles, int64_t iters, int forced_units)
{
    SkSplit sp;
    int64_t dp = tiles / kNumCUs * kNumCUs, rest = tiles - dp;
    if (rest == 0) {       // whole rounds: the last one as units of one tile each
        dp -= kNumCUs;
        rest = kNumCUs;
    }
    const int64_t total = rest * iters;
    const int64_t want = forced_units > 0 ? forced_units : kSkMaxUnits;
    sp.dp_tiles = int(dp);
    sp.units = int(std::min<int64_t>({want, kSkMaxUnits, total}));
    return sp;
}

// Stream-K workspace per (device, stream): two fp32 partial tiles per unit and
// one arrival counter per split tile, counters zeroed once at allocation (the
// kernel returns each to zero).  Calls on one stream are ordered, so they can
// share it; calls on different streams get different ones.  Allocated on a
// stream's first stream-K call, never while the stream is being captured into
// a graph (the call then uses whole tiles), and kept until the process ends.
constexpr size_t kSkFlagBytes = 4 * kNumCUs;
constexpr size_t kSkSlotBytes = size_t(256) * 256 * 4;
constexpr size_t kSkWsBytes = kSkFlagBytes + 2 * size_t(kSkMaxUnits) * kSkSlotBytes;
constexpr int kSkMaxPerDevice = 16;

struct SkWorkspace {
    int dev;
    hipStream_t stream;
    unsigned char* base;
};
std::mutex g_ws_mu;
std::vector<SkWorkspace> g_ws;

unsigned char* sk_workspace(int dev, hipStream_t st)
{
    // never under graph capture, even where the stream already has one: a
    // captured graph replayed on another stream would share it with this one
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return nullptr;
    std::lock_guard<std::mutex> lk(g_ws_mu);
    int on_dev = 0;
    for (const SkWorkspace& w : g_ws) {
        if (w.dev == dev && w.stream == st) return w.base;
        on_dev += w.dev == dev;
    }
    if (on_dev >= kSkMaxPerDevice) return nullptr;
    // Relaxed capture mode for this thread around the allocation, so that a
    // graph capture in global mode on another thread is not invalidated by it.
    void* p = nullptr;
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    const bool swapped = hipThreadExchangeStreamCaptureMode(&mode) == hipSuccess;
    const hipError_t merr = hipMalloc(&p, kSkWsBytes);
    if (swapped) (void)hipThreadExchangeStreamCaptureMode(&mode);
    if (merr != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (hipMemsetAsync(p, 0, kSkFlagBytes, st) != hipSuccess) {
        (void)hipFree(p);
        return nullptr;
    }
    g_ws.push_back({dev, st, static_cast<unsigned char*>(p)});
    return static_cast<unsigned char*>(p);
}

// A direct-copy configuration needs its 32-bit copy offsets to fit (a tile's
// rows of A or transposed B span BM * K * 2 bytes; a (K,N) B step spans
// BK * N * 2 bytes) and, for a (K,N) B, at least one full tile of columns: the
// last tile column is moved back to end at N.  Any 2-byte alignment is fine.
bool direct_fits(int id, int64_t N, int64_t K, int transB)
{
    const ConfigInfo& ci = config_info(id);
    if (!ci.direct) return true;
    if (K > (int64_t(1) << 22) || N > (int64_t(1) << 24)) return false;
    return transB || N >= ci.bn;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr const char* kSplitName = "d256x256x32_s4_i16+d256x192x32_s4_i16";
constexpr const char* kSplitName8 = "d256x256x32_s4_i16w8+d128x384x32_s4_i16w8";

// ---- two-region grid (16-bit inputs, B stored (N,K)): when whole rounds of
// 256x256 tiles over the CUs leave a partial round, the first `c` tile columns
// (c * tiles_m = whole rounds) stay 256x256 and the remaining columns are cut
// into narrower tiles of 3/4 the area, at most one round of them: 256x192
// tiles of four waves, in a grid whose first region is the four-wave 256x256
// tile, or (`eight`, only when forced) 128x384 tiles of eight waves behind the
// eight-wave 256x256 tile.  Measured on MI355X (bf16 4096x7168x4096, fp32 C)
// the four-wave grid takes 182.4 us, the eight-wave one 187.7 and eight-wave
// whole tiles 186.4: the 128x384 round runs at 0.74 of the 256x256 tile's
// rate per flop (each A fragment read by all eight waves), the 256x192 one at
// 0.81.  kSplitEff prices that round.
constexpr double kSplitEff = 0.93;

bool plan_split(Plan& p, int64_t M, int64_t N, int forced_cols, bool eight)
{
    const int cfg2 = eight ? CFG_D128x384x32_S4_I16W8 : CFG_D256x192x32_S4_I16;
    if (!config_built(cfg2)) return false;
    const int64_t bm2 = config_info(cfg2).bm, bn2 = config_info(cfg2).bn;
    const int64_t tm = p.tiles_m, tn = p.tiles_n, tiles = tm * tn;
    int64_t c = -1;
    if (forced_cols >= 0) {
        c = forced_cols;
    } else {
        const int64_t full = tiles / kNumCUs;
        if (full < 1 || tiles % kNumCUs == 0 || (full * kNumCUs) % tm != 0) return false;
        c = full * kNumCUs / tm;
    }
    if (c <= 0 || c >= tn) return false;
    const int64_t n_org = c * 256, w2 = N - n_org;
    const int64_t tn2 = ceil_div(w2, bn2), tiles2 = ceil_div(M, bm2) * tn2;
    if (forced_cols < 0) {
        const double plain = double(ceil_div(tiles, kNumCUs));
        const double split = double(c * tm / kNumCUs) +
                             double(ceil_div(tiles2, kNumCUs)) * (double(bm2 * bn2) / 65536.0) / kSplitEff;
        if (split >= 0.95 * plain) return false;
    }
    if (c * tm + tiles2 > INT32_MAX) return false;
    p.cfg2 = cfg2;
    p.tiles1 = int(c * tm);
    p.tiles_n = int(c);
    p.tiles_m2 = int(ceil_div(M, bm2));
    p.tiles_n2 = int(tn2);
    p.n_org2 = int(n_org);
    return true;
}

// ptrs = false: the choice for the sizes and codes alone (workspace queries),
// with no operand pointers to check.
Plan make_plan(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K,
               int in_dt, int out_dt, int transB, const Env& e, bool sk_ok = true, bool ptrs = true)
{
    Plan p;
    const int64_t lim = INT32_MAX;
    if (M < 0 || N < 0 || K < 0 || M > lim || N > lim || K > lim) {
        p.status = GEMM_RELU_EINVAL;
        return p;
    }
    if ((in_dt != GEMM_RELU_F16 && in_dt != GEMM_RELU_BF16 && !fp8_input(in_dt)) ||
        (out_dt != GEMM_RELU_F16 && out_dt != GEMM_RELU_BF16 && out_dt != GEMM_RELU_F32) ||
        (transB != 0 && transB != 1)) {
        p.status = GEMM_RELU_EINVAL;
        return p;
    }
    if (M == 0 || N == 0) {
        p.empty = true;
        return p;
    }
    const uint64_t in_bytes = uint64_t(elem_bytes(in_dt));
    const uint64_t a_bytes = uint64_t(M) * uint64_t(K) * in_bytes;
    const uint64_t b_bytes = uint64_t(K) * uint64_t(N) * in_bytes;
    const uint64_t c_bytes = uint64_t(M) * uint64_t(N) * uint64_t(elem_bytes(out_dt));
    if (ptrs && ((a_bytes && !A) || (b_bytes && !B) || !C)) {
        p.status = GEMM_RELU_EINVAL;
        return p;
    }
    if (ptrs && ((reinterpret_cast<uintptr_t>(A) & uintptr_t(in_bytes - 1)) ||
                 (reinterpret_cast<uintptr_t>(B) & uintptr_t(in_bytes - 1)) ||
                 (reinterpret_cast<uintptr_t>(C) & uintptr_t(elem_bytes(out_dt) - 1)))) {
        p.status = GEMM_RELU_EINVAL;
        return p;
    }
    const uintptr_t ua = reinterpret_cast<uintptr_t>(A), ub = reinterpret_cast<uintptr_t>(B),
                    uc = reinterpret_cast<uintptr_t>(C);
    if (ptrs && (overlaps(uc, c_bytes, ua, a_bytes) || overlaps(uc, c_bytes, ub, b_bytes))) {
        p.status = GEMM_RELU_EINVAL;
        return p;
    }

    auto tiles = [&](int id) { return ceil_div(M, config_info(id).bm) * ceil_div(N, config_info(id).bn); };
    // K steps of the 256x256x32 tile (64 elements a step for 8-bit inputs);
    // a stream-K split needs at least two
    const int64_t sk_iters = ceil_div(K, fp8_input(in_dt) ? 64 : 32);
    const bool sk_possible = sk_ok && sk_iters >= 2;
    auto usable = [&](int id) {
        return id != CFG_D256x128x64_S2 &&             // built for block-scaled inputs only
               !config_info(id).splitk &&               // needs a workspace (plan_splitk)
               ((id != CFG_D256x192x32_S4_I16 && id != CFG_D128x384x32_S4_I16W8) ||
                transB) &&                              // built for B stored (N,K) only
               // the persistent 16x16-block stream: whole 256x256 tiles inside
               // the matrix, whole K steps, at least a full ring of them
               (id != CFG_D256x256x32_S4_I16P || (M >= 256 && N >= 256 && K % 32 == 0 && K >= 128)) &&
               config_built(id) &&
               (id != CFG_D256x256x32_S4_ISK || sk_possible) &&
               id != CFG_D256x256x32_S4_I16W8SK &&      // needs a workspace (plan_streamk)
               direct_fits(id, N, K, transB) && (!fp8_input(in_dt) || fp8_config(id));
    };
    // Estimated time of a direct configuration, per K: rounds of workgroups
    // over the CUs, each round the longer of the tile's MFMA time (tile area
    // over its efficiency relative to the 256x256 tile, measured on MI355X:
    // 128x128 ~0.57, 64x64 ~0.5, the two-wave 64x32 tile ~0.25) and the time
    // to stream its (BM + BN) x K operands into one CU (~50 GB/s per CU from
    // beyond L2, i.e. 98 area units per row or column).
    auto cost = [&](int id) {
        const ConfigInfo& ci = config_info(id);
        const double eff = ci.bm >= 256 ? 1.0 : ci.bm >= 128 ? 0.57 : ci.bn >= 64 ? 0.5 : 0.25;
        const double per_round = std::max(ci.bm * ci.bn / eff, 98.0 * (ci.bm + ci.bn));
        return double(ceil_div(tiles(id), kNumCUs)) * per_round;
    };
    int cfg = -1;
    const int forced = e.force_cfg;
    if (forced >= 0 && usable(forced)) {
        cfg = forced;
    } else {
        // The 32x64 tile costs what the 64x32 one does under this model; measured
        // on MI355X it streams (K,N) B faster (whole 128-byte lines per k row) and
        // wins where M <= 64 and 64x64 tiles would leave half the CUs idle
        // (64x8192x8192: 28.0 vs 30.1 us; 64x4096x16384: 45.1 vs 50.1 us).  Where
        // 64x64 tiles fill the CUs they stream faster still (32x16384x8192: 41.7
        // vs 45.9 us), so it is not a candidate there.
        const bool skinny = M <= 64 && tiles(CFG_D64x64x64_S4) * 2 <= kNumCUs;
        // The 256x256 tile: 16x16x32 MFMA blocks for 16-bit inputs, which on
        // random data the power-limited chip clocks higher than the 32x32x16
        // form (measured 5-8% faster per call at 4096^3 and 8192^3, the same
        // bits), with eight waves; 8-bit inputs have only the 32x32x64 form here.
        const int big = fp8_input(in_dt) ? CFG_D256x256x32_S4_I : CFG_D256x256x32_S4_I16W8;
        for (int id : {big, int(CFG_D128x128x64_S3), int(CFG_D64x64x64_S4), int(CFG_D32x64x128_S4),
                       int(CFG_D64x32x128_S4)})
            if (usable(id) && (id != CFG_D32x64x128_S4 || skinny) && (cfg < 0 || cost(id) < cost(cfg)))
                cfg = id;
        if (cfg < 0) cfg = tiles(CFG_G128x128x64) >= kNumCUs ? CFG_G128x128x64 : CFG_G64x64x64;
    }
    // GEMM_RELU_SPLIT_COLS=<c> > 0 forces the two-region grid wherever it can
    // be built: behind the four-wave 256x256 tile, or behind the eight-wave one
    // when that is the forced configuration
    if (e.split_cols > 0 && transB && usable(CFG_D256x256x32_S4_I16) && forced != CFG_D256x256x32_S4_I16W8)
        cfg = CFG_D256x256x32_S4_I16;
    const int64_t tm = ceil_div(M, config_info(cfg).bm), tn = ceil_div(N, config_info(cfg).bn);
    if (tm * tn > lim) {
        p.status = GEMM_RELU_EUNSUPPORTED;
        return p;
    }
    p.cfg = cfg;
    p.tiles_m = int(tm);
    p.tiles_n = int(tn);
    // a narrower last round for 16-bit inputs with B stored (N,K): chosen by
    // the cost model unless a configuration was forced; GEMM_RELU_SPLIT_COLS
    // forces (or, with 0, forbids) it
    if ((cfg == CFG_D256x256x32_S4_I16 || cfg == CFG_D256x256x32_S4_I16W8) && transB && e.split_cols != 0 &&
        (e.split_cols > 0 || forced < 0))
        plan_split(p, M, N, e.split_cols > 0 ? e.split_cols : -1,
                   e.split_cols > 0 && forced == CFG_D256x256x32_S4_I16W8);
    if (config_info(cfg).streamk) {
        const SkSplit sp = sk_split(tm * tn, sk_iters, e.sk_units);
        p.dp_tiles = sp.dp_tiles;
        p.sk_units = sp.units;
    }
    return p;
}

// ---- K split with a workspace (gemm_relu_ws).  Skinny shapes (M <= 64) whose
// 64 x 128 tiles fill at most half the CUs: each tile's K steps are cut into
// `splits` equal parts, one workgroup each, enough to give every CU a part,
// with at least 8 steps a part.  With B stored (N,K) the workspace-free 32 x 64
// tiles already read whole K runs of each B row; there the split is taken only
// where those tiles would leave half the CUs idle (measured on MI355X, 64 x
// 8192 x 8192 fp16 from cold HBM: (K,N) B 40.4 -> 32.1 us per call; (N,K) B
// 34.1 -> 35.8 us, so not split).  GEMM_RELU_FORCE_CONFIG=d64x128x64_s4_splitk
// takes it for any shape of at most kSplitkMaxTiles tiles (up to 16 parts);
// GEMM_RELU_SPLITK_PARTS sets the part count.  Needs ws_need <= ws_bytes;
// otherwise the plan is left as it is.
// Workspace: kSplitkFlagBytes of arrival counters (one per tile, zero between
// calls), then splits x tiles fp32 partial tiles.
constexpr int kSplitkMaxParts = 16;
constexpr int kSplitkMaxTiles = 1024;
constexpr uint64_t kSplitkFlagBytes = 4 * kSplitkMaxTiles;

bool plan_splitk(Plan& p, int64_t M, int64_t N, int64_t K, int in_dt, int transB, uint64_t ws_bytes,
                 const Env& e)
{
    const bool forced = e.force_cfg >= 0 && config_info(e.force_cfg).splitk;
    if (e.force_cfg >= 0 && !forced) return false;
    const int id = forced ? e.force_cfg : int(CFG_D64x128x64_S4_SPLITK);
    const ConfigInfo& ci = config_info(id);
    if (ws_bytes == 0 || !config_built(id) || !direct_fits(id, N, K, transB)) return false;
    const int64_t steps = ceil_div(K, fp8_input(in_dt) ? 2 * ci.bk16 : ci.bk16);
    const int64_t tiles = ceil_div(M, ci.bm) * ceil_div(N, ci.bn);
    const int64_t slots = int64_t(kNumCUs) * ci.per_cu;      // workgroups resident at once
    int64_t parts = 0;
    if (e.splitk_parts > 0 && (forced || M <= 64)) {
        parts = e.splitk_parts;
    } else if (forced) {
        parts = std::max<int64_t>(2, std::min<int64_t>(kSplitkMaxParts, slots / tiles));
    } else {
        if (M > 64 || tiles * 2 > kNumCUs) return false;
        if (transB && ceil_div(M, 32) * ceil_div(N, 64) * 2 > kNumCUs) return false;
        parts = std::min<int64_t>({kSplitkMaxParts, slots / tiles, steps / 8});
    }
    parts = std::min<int64_t>({parts, steps, kSplitkMaxParts});
    if (parts < 2) return false;
    const int64_t split_steps = ceil_div(steps, parts);
    const int64_t splits = ceil_div(steps, split_steps);     // every part non-empty
    if (splits < 2 || tiles > kSplitkMaxTiles) return false;
    const uint64_t need = kSplitkFlagBytes + uint64_t(splits) * uint64_t(tiles) * ci.bm * ci.bn * 4;
    if (need > ws_bytes) return false;
    p.cfg = id;
    p.cfg2 = -1;
    p.tiles_m = int(ceil_div(M, ci.bm));
    p.tiles_n = int(ceil_div(N, ci.bn));
    p.splits = int(splits);
    p.split_steps = int(split_steps);
    p.ws_need = need;
    return true;
}

// ---- stream-K with a workspace (gemm_relu_ws; the eight-wave tile's
// comparison configuration, taken only when GEMM_RELU_FORCE_CONFIG names it):
// whole rounds keep one workgroup per tile and the rest of the tiles' K steps
// are shared equally by one workgroup per CU, or GEMM_RELU_SK_UNITS of them.
// Each split tile has an arrival counter in the workspace's first 4096 bytes;
// the fp32 partials follow, two 256 KiB slots per unit.  Measured on MI355X
// it loses to whole tiles wherever it applies (the exchange of 256 KiB
// partials through device-coherent memory costs more than the partly empty
// last round), so plan selection never takes it.
constexpr uint64_t kSkSlotFloats = 256 * 256;

bool plan_streamk(Plan& p, int64_t M, int64_t N, int64_t K, int in_dt, int transB, uint64_t ws_bytes,
                  const Env& e)
{
    const int id = CFG_D256x256x32_S4_I16W8SK;
    if (e.force_cfg != id) return false;
    if (ws_bytes == 0 || fp8_input(in_dt) || !config_built(id) || !direct_fits(id, N, K, transB)) return false;
    const int64_t tiles = ceil_div(M, 256) * ceil_div(N, 256);
    const int64_t iters = ceil_div(K, 32);
    const int64_t rest = tiles % kNumCUs;
    if (rest == 0 || tiles > INT32_MAX) return false;
    const SkSplit sp = sk_split(tiles, iters, e.sk_units);
    if (sp.units < 1) return false;
    if (rest > int64_t(kSplitkFlagBytes / 4)) return false;
    const uint64_t need = kSplitkFlagBytes + 2 * uint64_t(sp.units) * kSkSlotFloats * 4;
    if (need > ws_bytes) return false;
    p.cfg = id;
    p.cfg2 = -1;
    p.tiles_m = int(ceil_div(M, 256));
    p.tiles_n = int(ceil_div(N, 256));
    p.dp_tiles = sp.dp_tiles;
    p.sk_units = sp.units;
    p.ws_need = need;
    return true;
}

// ---- block-scaled (MX) inputs
bool mx_format(int f) { return f == GEMM_RELU_MX_E4M3 || f == GEMM_RELU_MX_E5M2 || f == GEMM_RELU_MX_E2M1; }

Plan make_plan_mx(const void* A, const void* SA, const void* B, const void* SB, const void* C,
                  int64_t M, int64_t N, int64_t K, int fmt, int out_dt, const Env& e)
{
    Plan p;
    const int64_t lim = INT32_MAX;
    if (M < 0 || N < 0 || K < 0 || M > lim || N > lim || K > lim || K % 32 != 0 ||
        !mx_format(fmt) ||
        (out_dt != GEMM_RELU_F16 && out_dt != GEMM_RELU_BF16 && out_dt != GEMM_RELU_F32)) {
        p.status = GEMM_RELU_EINVAL;
        return p;
    }
    if (M == 0 || N == 0) {
        p.empty = true;
        return p;
    }
    const int64_t ks = fmt == GEMM_RELU_MX_E2M1 ? K / 2 : K;     // storage bytes per row
    const uint64_t a_bytes = uint64_t(M) * uint64_t(ks), b_bytes = uint64_t(N) * uint64_t(ks);
    const uint64_t sa_bytes = uint64_t(M) * uint64_t(K / 32), sb_bytes = uint64_t(N) * uint64_t(K / 32);
    const uint64_t c_bytes = uint64_t(M) * uint64_t(N) * uint64_t(elem_bytes(out_dt));
    if ((a_bytes && (!A || !SA)) || (b_bytes && (!B || !SB)) || !C ||
        (reinterpret_cast<uintptr_t>(C) & uintptr_t(elem_bytes(out_dt) - 1))) {
        p.status = GEMM_RELU_EINVAL;
        return p;
    }
    const uintptr_t uc = reinterpret_cast<uintptr_t>(C);
    if (overlaps(uc, c_bytes, reinterpret_cast<uintptr_t>(A), a_bytes) ||
        overlaps(uc, c_bytes, reinterpret_cast<uintptr_t>(B), b_bytes) ||
        overlaps(uc, c_bytes, reinterpret_cast<uintptr_t>(SA), sa_bytes) ||
        overlaps(uc, c_bytes, reinterpret_cast<uintptr_t>(SB), sb_bytes)) {
        p.status = GEMM_RELU_EINVAL;
        return p;
    }
    // The interleaved pipeline stages scales in LDS by 16-byte row pieces (so
    // rows of at least 16 blocks) and addresses them with 32-bit offsets.
    const bool lds_scales_fit = K / 32 >= 16 && sa_bytes < (uint64_t(1) << 32) &&
                                sb_bytes < (uint64_t(1) << 32);
    auto usable = [&](int id) {
        return (id == CFG_D256x256x64_S2 || id == CFG_D256x128x64_S2 || id == CFG_D128x128x64_S2 ||
                (id == CFG_D256x256x32_S4_I && lds_scales_fit)) &&
               config_built(id) && direct_fits(id, N, ks, 1);
    };
    // Estimated time per K, as for the other inputs: rounds of workgroups over
    // the CUs times the tile's area over its efficiency relative to the
    // interleaved 256x256 tile (the two-stage 128x128 tile measured 0.59
    // (MXFP8) and 0.74 (MXFP4) of it at 8192^3).  The two-stage 256x256 and
    // 256x128 tiles stay selectable for comparison.
    auto tiles = [&](int id) { return ceil_div(M, config_info(id).bm) * ceil_div(N, config_info(id).bn); };
    auto cost = [&](int id) {
        const ConfigInfo& ci = config_info(id);
        return double(ceil_div(tiles(id), kNumCUs)) * ci.bm * ci.bn / (ci.bm >= 256 ? 1.0 : 0.6);
    };
    int cfg = -1;
    if (e.force_cfg >= 0 && usable(e.force_cfg)) {
        cfg = e.force_cfg;
    } else {
        for (int id : {CFG_D256x256x32_S4_I, CFG_D128x128x64_S2})
            if (usable(id) && (cfg < 0 || cost(id) < cost(cfg))) cfg = id;
    }
    if (cfg < 0) {
        p.status = GEMM_RELU_EUNSUPPORTED;     // K beyond the 32-bit copy offsets
        return p;
    }
    const int64_t tm = ceil_div(M, config_info(cfg).bm), tn = ceil_div(N, config_info(cfg).bn);
    if (tm * tn > lim) {
        p.status = GEMM_RELU_EUNSUPPORTED;
        return p;
    }
    p.cfg = cfg;
    p.tiles_m = int(tm);
    p.tiles_n = int(tn);
    return p;
}

// ---- 2:4 sparse A
// 2 x 4 waves (variant 1); the 2 x 2-wave variant 0 is a comparison build's, by name
constexpr const char* kSpConfigName = "sp256x256x64_s3_w8";
constexpr const char* kSpW4Name = "sp256x256x64_s3";
constexpr int kSpTile = 256;

Plan make_plan_sp(const void* As, const void* E, const void* B, const void* C, int64_t M,
                  int64_t N, int64_t K, int in_dt, int out_dt, int transB)
{
    Plan p;
    const int64_t lim = INT32_MAX;
    if (M < 0 || N < 0 || K < 0 || M > lim || N > lim || K > lim || K % 4 != 0 ||
        (in_dt != GEMM_RELU_F16 && in_dt != GEMM_RELU_BF16) ||
        (out_dt != GEMM_RELU_F16 && out_dt != GEMM_RELU_BF16 && out_dt != GEMM_RELU_F32) ||
        (transB != 0 && transB != 1)) {
        p.status = GEMM_RELU_EINVAL;
        return p;
    }
    if (M == 0 || N == 0) {
        p.empty = true;
        return p;
    }
    const uint64_t as_bytes = uint64_t(M) * uint64_t(K / 2) * 2;
    const uint64_t e_bytes = uint64_t((K + 63) / 64) * uint64_t(M) * 8;
    const uint64_t b_bytes = uint64_t(K) * uint64_t(N) * 2;
    const uint64_t c_bytes = uint64_t(M) * uint64_t(N) * uint64_t(elem_bytes(out_dt));
    const uintptr_t ua = reinterpret_cast<uintptr_t>(As), ub = reinterpret_cast<uintptr_t>(B);
    const uintptr_t uc = reinterpret_cast<uintptr_t>(C), ue = reinterpret_cast<uintptr_t>(E);
    if ((as_bytes && (!As || !E)) || (b_bytes && !B) || !C || (ua & 1) || (ub & 1) ||
        (uc & uintptr_t(elem_bytes(out_dt) - 1))) {
        p.status = GEMM_RELU_EINVAL;
        return p;
    }
    if (overlaps(uc, c_bytes, ua, as_bytes) || overlaps(uc, c_bytes, ue, e_bytes) ||
        overlaps(uc, c_bytes, ub, b_bytes)) {
        p.status = GEMM_RELU_EINVAL;
        return p;
    }
    // 32-bit copy offsets (a tile's rows span 256 * K * 2 bytes, a (K,N) B step
    // 64 * N * 2), and a (K,N) B needs one full tile of columns
    if (K > (int64_t(1) << 22) || N > (int64_t(1) << 24) || (!transB && N < kSpTile)) {
        p.status = GEMM_RELU_EUNSUPPORTED;
        return p;
    }
    const int64_t tm = ceil_div(M, kSpTile), tn = ceil_div(N, kSpTile);
    if (tm * tn > lim) {
        p.status = GEMM_RELU_EUNSUPPORTED;
        return p;
    }
    const char* f = std::getenv("GEMM_RELU_FORCE_CONFIG");
    p.cfg = kComparisonBuilt && f && std::strcmp(f, kSpW4Name) == 0 ? 0 : 1;
    p.tiles_m = int(tm);
    p.tiles_n = int(tn);
    return p;
}

LaunchFn pick_launcher_mx(int fmt, int out_dt, int cfg)
{
    switch (fmt) {
    case GEMM_RELU_MX_E4M3: return launcher_mx_e4m3(out_dt, cfg);
    case GEMM_RELU_MX_E5M2: return launcher_mx_e5m2(out_dt, cfg);
    case GEMM_RELU_MX_E2M1: return launcher_mx_e2m1(out_dt, cfg);
    default: return nullptr;
    }
}

LaunchFn pick_launcher(int in_dt, int out_dt, int transB, int cfg)
{
    switch (in_dt) {
    case GEMM_RELU_F16: return transB ? launcher_f16_nt(out_dt, cfg) : launcher_f16_nn(out_dt, cfg);
    case GEMM_RELU_BF16: return transB ? launcher_bf16_nt(out_dt, cfg) : launcher_bf16_nn(out_dt, cfg);
    case GEMM_RELU_F8_E4M3:
        return transB ? launcher_f8e4m3_nt(out_dt, cfg) : launcher_f8e4m3_nn(out_dt, cfg);
    case GEMM_RELU_F8_E5M2:
        return transB ? launcher_f8e5m2_nt(out_dt, cfg) : launcher_f8e5m2_nn(out_dt, cfg);
    default: return nullptr;
    }
}

// A caller's workspace: NULL or 0 bytes means none; otherwise 256-byte aligned
// and disjoint from A, B and C.
bool workspace_ok(const void* ws, uint64_t ws_bytes, const void* A, const void* B, const void* C,
                  int64_t M, int64_t N, int64_t K, int in_dt, int out_dt)
{
    if (!ws || ws_bytes == 0) return true;
    const uintptr_t uw = reinterpret_cast<uintptr_t>(ws);
    if (uw & 255) return false;
    const uint64_t in_bytes = uint64_t(elem_bytes(in_dt));
    return !overlaps(uw, ws_bytes, reinterpret_cast<uintptr_t>(A), uint64_t(M) * uint64_t(K) * in_bytes) &&
           !overlaps(uw, ws_bytes, reinterpret_cast<uintptr_t>(B), uint64_t(K) * uint64_t(N) * in_bytes) &&
           !overlaps(uw, ws_bytes, reinterpret_cast<uintptr_t>(C),
                     uint64_t(M) * uint64_t(N) * uint64_t(elem_bytes(out_dt)));
}

// The plan of gemm_relu / gemm_relu_ws: the workspace-free choice, then a K
// split where a workspace of ws_bytes allows one.
Plan make_plan_ws(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K, int in_dt,
                  int out_dt, int transB, const void* ws, uint64_t ws_bytes, const Env& e)
{
    Plan p = make_plan(A, B, C, M, N, K, in_dt, out_dt, transB, e);
    if (p.status != GEMM_RELU_OK || p.empty) return p;
    if (!workspace_ok(ws, ws_bytes, A, B, C, M, N, K, in_dt, out_dt)) {
        p.status = GEMM_RELU_EINVAL;
        return p;
    }
    if (ws && ws_bytes && !plan_splitk(p, M, N, K, in_dt, transB, ws_bytes, e))
        plan_streamk(p, M, N, K, in_dt, transB, ws_bytes, e);
    return p;
}

int run_gemm_relu(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int in_dtype,
                  int out_dtype, int transB, void* workspace, uint64_t ws_bytes, void* stream)
{
    const Env e = env();
    Plan p = make_plan_ws(A, B, C, M, N, K, in_dtype, out_dtype, transB, workspace, ws_bytes, e);
    if (p.status != GEMM_RELU_OK) return p.status;
    if (p.empty) return GEMM_RELU_OK;
    const int dev = check_device();
    if (dev != GEMM_RELU_OK) return dev;
    hipStream_t st = static_cast<hipStream_t>(stream);
    unsigned char* ws = nullptr;
    if (config_info(p.cfg).streamk && p.ws_need > 0) {
        ws = static_cast<unsigned char*>(workspace);       // the caller's (plan_streamk)
    } else if (config_info(p.cfg).streamk) {
        int d = 0;
        if (hipGetDevice(&d) != hipSuccess) return GEMM_RELU_EHIP;
        ws = sk_workspace(d, st);
        if (!ws) p = make_plan(A, B, C, M, N, K, in_dtype, out_dtype, transB, e, false);
    }

    KernelArgs args{};
    args.A = static_cast<const unsigned char*>(A);
    args.B = static_cast<const unsigned char*>(B);
    args.C = static_cast<unsigned char*>(C);
    args.M = int(M);
    args.N = int(N);
    args.K = int(K);
    args.tiles_m = p.tiles_m;
    args.tiles_n = p.tiles_n;
    const int panel = e.panel > 0 ? e.panel : 8;
    args.panel = panel < p.tiles_m ? panel : p.tiles_m;
    args.nxcd = e.nxcd;
    args.SA = nullptr;
    args.SB = nullptr;
    args.KB = 0;
    if (config_info(p.cfg).streamk) {
        args.flags = reinterpret_cast<unsigned*>(ws);
        args.ws = reinterpret_cast<float*>(ws + (p.ws_need > 0 ? kSplitkFlagBytes : kSkFlagBytes));
        args.dp_tiles = p.dp_tiles;
        args.sk_units = p.sk_units;
    }
    if (p.splits > 0) {
        args.flags = static_cast<unsigned*>(workspace);
        args.ws = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + kSplitkFlagBytes);
        args.splits = p.splits;
        args.split_steps = p.split_steps;
    }

    LaunchFn fn = p.cfg2 >= 0 ? launcher_i16_2r(in_dtype, out_dtype, p.cfg2)
                              : pick_launcher(in_dtype, out_dtype, transB, p.cfg);
    if (!fn) return GEMM_RELU_EUNSUPPORTED;
    const int tiles = p.tiles_m * p.tiles_n;
    int grid = config_info(p.cfg).persistent ? std::min(tiles, e.pgrid > 0 ? e.pgrid : kNumCUs)
               : config_info(p.cfg).streamk  ? p.dp_tiles + p.sk_units
               : p.splits > 0                ? tiles * p.splits
                                             : tiles;
    if (p.cfg2 >= 0) {
        args.tiles1 = p.tiles1;
        args.tiles_m2 = p.tiles_m2;
        args.tiles_n2 = p.tiles_n2;
        args.panel2 = panel < p.tiles_m2 ? panel : p.tiles_m2;
        args.n_org2 = p.n_org2;
        grid = p.tiles1 + p.tiles_m2 * p.tiles_n2;
    }
    if (fn(args, grid, st) != hipSuccess) return GEMM_RELU_EHIP;
    if (e.sync) {
        if (hipStreamSynchronize(st) != hipSuccess) return GEMM_RELU_EHIP;
        if (hipGetLastError() != hipSuccess) return GEMM_RELU_EHIP;
    }
    return GEMM_RELU_OK;
}

// ---- gemm_relu_noalloc: the K-split workspace in a device array of the
// library (one per GPU, held until the process ends) instead of the caller's.
// Host code never passes the array's name to a kernel: its device address is
// looked up once per device, with that device current.
constexpr uint64_t kScratchBytes = uint64_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchAddr {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchAddr g_scratch[kMaxDevices];

void* scratch_address(int dev)
{
    ScratchAddr& s = g_scratch[dev];
    std::call_once(s.once, [&] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
    return s.err == hipSuccess ? s.ptr : nullptr;
}

// Zeroes the arrival words at the start of the scratch (a kernel, so that a
// captured graph holds no memset node).
__global__ void __launch_bounds__(256) clear_words(unsigned* p, int n)
{
    for (int i = threadIdx.x; i < n; i += 256) p[i] = 0u;
}

bool codes_and_sizes_ok(int64_t M, int64_t N, int64_t K, int in_dt, int out_dt, int transB)
{
    const int64_t lim = INT32_MAX;
    return M >= 0 && N >= 0 && K >= 0 && M <= lim && N <= lim && K <= lim &&
           (in_dt == GEMM_RELU_F16 || in_dt == GEMM_RELU_BF16 || fp8_input(in_dt)) &&
           (out_dt == GEMM_RELU_F16 || out_dt == GEMM_RELU_BF16 || out_dt == GEMM_RELU_F32) &&
           (transB == 0 || transB == 1);
}

}  // namespace

extern "C" int gemm_relu(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                         int in_dtype, int out_dtype, int transB, void* stream)
{
    return run_gemm_relu(A, B, C, M, N, K, in_dtype, out_dtype, transB, nullptr, 0, stream);
}

extern "C" int gemm_relu_ws(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                            int in_dtype, int out_dtype, int transB, void* workspace,
                            uint64_t workspace_bytes, void* stream)
{
    return run_gemm_relu(A, B, C, M, N, K, in_dtype, out_dtype, transB, workspace, workspace_bytes,
                         stream);
}

extern "C" int gemm_relu_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                                 int in_dtype, int out_dtype, int transB, void* stream)
{
    const Env e = env();
    const Plan p = make_plan(A, B, C, M, N, K, in_dtype, out_dtype, transB, e);
    if (p.status != GEMM_RELU_OK) return p.status;
    if (p.empty) return GEMM_RELU_OK;
    Plan q = p;
    if (!plan_splitk(q, M, N, K, in_dtype, transB, UINT64_MAX, e))
        return run_gemm_relu(A, B, C, M, N, K, in_dtype, out_dtype, transB, nullptr, 0, stream);
    if (q.ws_need > kScratchBytes) return GEMM_RELU_ESCRATCH;
    const int dev = check_device();
    if (dev != GEMM_RELU_OK) return dev;
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess) return GEMM_RELU_EHIP;
    void* ws = scratch_address(d);
    if (!ws) return GEMM_RELU_EHIP;
    // the scratch keeps what the last call on this GPU left: start from
    // zeroed arrival words
    hipStream_t st = static_cast<hipStream_t>(stream);
    void* params[] = {&ws, const_cast<int*>(&kSplitkMaxTiles)};
    if (hipLaunchKernel(reinterpret_cast<const void*>(&clear_words), dim3(1), dim3(256), params, 0, st) !=
        hipSuccess)
        return GEMM_RELU_EHIP;
    return run_gemm_relu(A, B, C, M, N, K, in_dtype, out_dtype, transB, ws, kScratchBytes, stream);
}

extern "C" int64_t gemm_relu_workspace_size(int64_t M, int64_t N, int64_t K, int in_dtype, int out_dtype,
                                            int transB)
{
    if (!codes_and_sizes_ok(M, N, K, in_dtype, out_dtype, transB)) return GEMM_RELU_EINVAL;
    if (M == 0 || N == 0) return 0;
    const Env e = env();
    Plan p;
    if (plan_splitk(p, M, N, K, in_dtype, transB, UINT64_MAX, e)) return int64_t(p.ws_need);
    // stream-K (forced only) on top of what plan selection takes without one
    p = make_plan(nullptr, nullptr, nullptr, M, N, K, in_dtype, out_dtype, transB, e, true, false);
    if (!plan_streamk(p, M, N, K, in_dtype, transB, UINT64_MAX, e)) return 0;
    return int64_t(p.ws_need);
}

extern "C" const char* gemm_relu_configs(void)
{
    static const std::string names = [] {
        std::string out;
        for (int id = 0; id < CFG_COUNT; ++id)
            if (config_built(id)) {
                if (!out.empty()) out += ',';
                out += config_info(id).name;
            }
        out += ',';
        out += kSplitName;
        if (config_built(CFG_D128x384x32_S4_I16W8)) {
            out += ',';
            out += kSplitName8;
        }
        out += ',';
        out += kSpConfigName;
        if (kComparisonBuilt) {
            out += ',';
            out += kSpW4Name;
        }
        return out;
    }();
    return names.c_str();
}

extern "C" const char* gemm_relu_strerror(int status)
{
    switch (status) {
    case GEMM_RELU_OK: return "success";
    case GEMM_RELU_EINVAL: return "invalid argument";
    case GEMM_RELU_EUNSUPPORTED: return "unsupported device or size";
    case GEMM_RELU_EHIP: return "HIP runtime error";
    case GEMM_RELU_ESCRATCH: return "the K split needs more than the 16 MiB scratch of gemm_relu_noalloc";
    default: return "unknown status";
    }
}

static const char* plan_name(const Plan& p)
{
    if (p.cfg2 < 0) return config_info(p.cfg).name;
    return p.cfg2 == CFG_D128x384x32_S4_I16W8 ? kSplitName8 : kSplitName;
}

extern "C" const char* gemm_relu_plan(const void* A, const void* B, const void* C, int64_t M,
                                      int64_t N, int64_t K, int in_dtype, int out_dtype,
                                      int transB)
{
    const Plan p = make_plan(A, B, C, M, N, K, in_dtype, out_dtype, transB, env());
    if (p.status == GEMM_RELU_EINVAL) return nullptr;
    if (p.status != GEMM_RELU_OK) return "unsupported";
    if (p.empty) return "none";
    return plan_name(p);
}

extern "C" const char* gemm_relu_ws_plan(const void* A, const void* B, const void* C, int64_t M, int64_t N,
                                         int64_t K, int in_dtype, int out_dtype, int transB,
                                         const void* workspace, uint64_t workspace_bytes)
{
    const Plan p = make_plan_ws(A, B, C, M, N, K, in_dtype, out_dtype, transB, workspace, workspace_bytes,
                                env());
    if (p.status == GEMM_RELU_EINVAL) return nullptr;
    if (p.status != GEMM_RELU_OK) return "unsupported";
    if (p.empty) return "none";
    return plan_name(p);
}

extern "C" int gemm_relu_mx(const void* A, const void* SA, const void* B, const void* SB, void* C,
                            int64_t M, int64_t N, int64_t K, int fmt, int out_dtype, void* stream)
{
    const Env e = env();
    const Plan p = make_plan_mx(A, SA, B, SB, C, M, N, K, fmt, out_dtype, e);
    if (p.status != GEMM_RELU_OK) return p.status;
    if (p.empty) return GEMM_RELU_OK;
    const int dev = check_device();
    if (dev != GEMM_RELU_OK) return dev;

    KernelArgs args{};
    args.A = static_cast<const unsigned char*>(A);
    args.B = static_cast<const unsigned char*>(B);
    args.C = static_cast<unsigned char*>(C);
    args.M = int(M);
    args.N = int(N);
    args.K = int(fmt == GEMM_RELU_MX_E2M1 ? K / 2 : K);     // storage bytes per row
    args.tiles_m = p.tiles_m;
    args.tiles_n = p.tiles_n;
    const int panel = e.panel > 0 ? e.panel : 8;
    args.panel = panel < p.tiles_m ? panel : p.tiles_m;
    args.nxcd = e.nxcd;
    args.SA = static_cast<const unsigned char*>(SA);
    args.SB = static_cast<const unsigned char*>(SB);
    args.KB = int(K / 32);

    LaunchFn fn = pick_launcher_mx(fmt, out_dtype, p.cfg);
    if (!fn) return GEMM_RELU_EUNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (fn(args, p.tiles_m * p.tiles_n, st) != hipSuccess) return GEMM_RELU_EHIP;
    if (e.sync) {
        if (hipStreamSynchronize(st) != hipSuccess) return GEMM_RELU_EHIP;
        if (hipGetLastError() != hipSuccess) return GEMM_RELU_EHIP;
    }
    return GEMM_RELU_OK;
}

extern "C" const char* gemm_relu_mx_plan(const void* A, const void* SA, const void* B,
                                         const void* SB, const void* C, int64_t M, int64_t N,
                                         int64_t K, int fmt, int out_dtype)
{
    const Plan p = make_plan_mx(A, SA, B, SB, C, M, N, K, fmt, out_dtype, env());
    if (p.status == GEMM_RELU_EINVAL) return nullptr;
    if (p.status != GEMM_RELU_OK) return "unsupported";
    if (p.empty) return "none";
    return config_info(p.cfg).name;
}

extern "C" int gemm_relu_sp(const void* As, const void* E, const void* B, void* C, int64_t M,
                            int64_t N, int64_t K, int in_dtype, int out_dtype, int transB,
                            void* stream)
{
    const Env e = env();
    const Plan p = make_plan_sp(As, E, B, C, M, N, K, in_dtype, out_dtype, transB);
    if (p.status != GEMM_RELU_OK) return p.status;
    if (p.empty) return GEMM_RELU_OK;
    const int dev = check_device();
    if (dev != GEMM_RELU_OK) return dev;

    SpArgs args;
    args.As = static_cast<const unsigned char*>(As);
    args.E = static_cast<const unsigned char*>(E);
    args.B = static_cast<const unsigned char*>(B);
    args.C = static_cast<unsigned char*>(C);
    args.M = int(M);
    args.N = int(N);
    args.K = int(K);
    args.tiles_m = p.tiles_m;
    args.tiles_n = p.tiles_n;
    const int panel = e.panel > 0 ? e.panel : 8;
    args.panel = panel < p.tiles_m ? panel : p.tiles_m;
    args.nxcd = e.nxcd;

    SpLaunchFn fn = launcher_sp(in_dtype, out_dtype, transB, p.cfg);
    if (!fn) return GEMM_RELU_EUNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (fn(args, p.tiles_m * p.tiles_n, st) != hipSuccess) return GEMM_RELU_EHIP;
    if (e.sync) {
        if (hipStreamSynchronize(st) != hipSuccess) return GEMM_RELU_EHIP;
        if (hipGetLastError() != hipSuccess) return GEMM_RELU_EHIP;
    }
    return GEMM_RELU_OK;
}

extern "C" const char* gemm_relu_sp_plan(const void* As, const void* E, const void* B,
                                         const void* C, int64_t M, int64_t N, int64_t K,
                                         int in_dtype, int out_dtype, int transB)
{
    const Plan p = make_plan_sp(As, E, B, C, M, N, K, in_dtype, out_dtype, transB);
    if (p.status == GEMM_RELU_EINVAL) return nullptr;
    if (p.status != GEMM_RELU_OK) return "unsupported";
    if (p.empty) return "none";
    return p.cfg == 1 ? kSpConfigName : kSpW4Name;
}
