// Host side of libwq: argument validation, device properties, options,
// per-shape plan and the C ABI declared in include/wq.h.
#include "wq.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "wq_internal.h"

namespace {

using wq::GemmArgs;

constexpr int kPackedFormatVersion = 3;
constexpr int kMaxDevices = 64;

// ----------------------------------------------------------------- options
struct Options {
    int force_path = WQ_PATH_AUTO;
    int nt = 0;              // 0 = per-shape choice
    int sn = 0;              // 0 = per-shape choice
    int split = 0;           // 0 = per-shape choice
    int waves_per_cu = 4;    // target resident waves per compute unit
    int kp = 0;              // K parts across work-groups with a workspace; 0 = per-shape choice
    int w8a8_stages = 0;     // W8A8 LDS pipeline depth (2 or 4); 0 = per-grid choice
};

Options g_opts;

const Options& options()
{
    static Options& o = g_opts;
    static std::once_flag once;
    std::call_once(once, [] {
        if (const char* p = std::getenv("WQ_FORCE_PATH")) {
            if (!std::strcmp(p, "gemv")) o.force_path = WQ_PATH_GEMV;
            else if (!std::strcmp(p, "mfma")) o.force_path = WQ_PATH_MFMA;
        }
        if (const char* p = std::getenv("WQ_NT")) {
            int v = std::atoi(p);
            if (v == 1 || v == 2) o.nt = v;
        }
        if (const char* p = std::getenv("WQ_SN")) {
            int v = std::atoi(p);
            if (v >= 1 && v <= 8) o.sn = v;
        }
        if (const char* p = std::getenv("WQ_SPLIT")) {
            int v = std::atoi(p);
            if (v >= 1 && v <= 16) o.split = v;
        }
        if (const char* p = std::getenv("WQ_WAVES_PER_CU")) {
            int v = std::atoi(p);
            if (v >= 1 && v <= 32) o.waves_per_cu = v;
        }
        if (const char* p = std::getenv("WQ_KPARTS")) {
            int v = std::atoi(p);
            if (v >= 1 && v <= wq::kMaxKParts) o.kp = v;
        }
    });
    return o;
}

// -------------------------------------------------------- device properties
struct DevInfo {
    bool ok = false;
    bool gfx950 = false;
    int cu = 0;
};

std::mutex g_dev_mu;
DevInfo g_dev[kMaxDevices];

// Returns WQ_OK and fills *info for the current device.
wq_status current_device(DevInfo* info, int* dev_out = nullptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return WQ_ERR_HIP;
    }
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DevInfo& d = g_dev[dev];
    if (!d.ok) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return WQ_ERR_HIP;
        }
        d.cu = prop.multiProcessorCount;
        d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        d.ok = true;
    }
    *info = d;
    if (dev_out) *dev_out = dev;
    return d.gfx950 ? WQ_OK : WQ_ERR_DEVICE;
}

// --------------------------------------------------------------------- plan
// A work-group covers SN*NT tiles of 16 output columns over all of K, or
// over one of KP K parts: SN column-waves (NT tiles each) share staged
// activation chunks, and SK K-groups split the work-group's K blocks (split =
// SN*SK waves).  Sharing cuts the activation reads (every work-group reads
// its part of x once), so a plan takes as many tiles per work-group as still
// leaves about one work-group per compute unit, and adds K groups where that
// leaves too few waves.  Without a workspace KP = 1 and every output is
// reduced inside its work-group.  With one, a low-N shape with a long K
// splits K across work-groups as well (KP > 1; atlas "Module m16_tc", "WHY
// THE FFN ARM LOSES": the low-N projections' grids against the machine's
// slots): each K part's work-group writes FP32 partials and a second kernel
// adds the parts in order, so the grid can cover the CUs without thinning the
// activation sharing.
struct Plan {
    int kind = 0;
    int nt = 1;
    int sn = 1;
    int split = 1;
    int kp = 1;
    int n_tiles = 0, n_cg = 0, KB = 0;
};

// Largest M the automatic ladder sends to the FP8 GEMV: none.  Both arms
// timed on one build (python bench.py --crossover; HIP graphs, weight copies
// rotated past the Infinity Cache), M = 1 / 2 / 3 / 4 in us, GEMV vs MFMA
// tile: FFN gate/up 16.8 / 21.2 / 27.0 / 32.9 vs 16.9 / 16.9 / 16.8 / 16.8;
// FFN down 19.8 / 26.7 / 33.6 / 40.3 vs 19.1 / 19.2 / 19.2 / 19.5; attention
// Q 9.3 / 10.6 / 12.4 / 14.3 vs 9.0 for every M; attention K/V 7.9 / 9.8 /
// 11.7 / 13.4 vs 6.5 / 6.6.  The tile's time does not change with M, the
// GEMV's FP32 FMAs grow with it, and at M = 1 the tile ties or wins (it also
// takes the shape's K-split plan).  So the first M at which the GEMV beats
// the better arm does not exist, and AUTO takes the tile for every M; the
// GEMV stays selectable (WQ_PATH_GEMV, WQ_FORCE_PATH=gemv) for M <= 4, for
// callers that want its strict K order.  (The arc PR, "The threshold": the
// crossover is a measured lever, taken from a sweep of all arms on one
// binary, not a constant of the method.)
constexpr int64_t kGemvAutoMaxM = 0;

// Tilings measured fastest on MI355X (256 CUs) for the decode shapes of the
// FFN and attention projections (a dispatch table chosen per shape from
// measurements, as the FLUTE PR's opening summary describes for its kernel);
// other shapes use the rule below.
struct TableEntry {
    int kind;
    int64_t N, K;
    int nt, sn, split;
    int kp;                  // K parts across work-groups (1: none)
};
constexpr TableEntry kTable[] = {
    {wq::KIND_MFMA_FP8, 17408, 5120, 1, 5, 5, 1},    // FFN gate/up
    {wq::KIND_MFMA_FP8, 5120, 17408, 1, 2, 6, 1},    // FFN down
    {wq::KIND_MFMA_FP8, 6144, 5120, 1, 2, 6, 1},     // attention Q
    {wq::KIND_MFMA_FP8, 1024, 5120, 1, 1, 4, 1},     // attention K, V
    {wq::KIND_MFMA_FP8, 8192, 5120, 1, 2, 6, 1},     // attention Q, K and V stacked in one matrix
    {wq::KIND_MFMA_FP8, 5120, 6144, 1, 2, 6, 1},     // attention output
    {wq::KIND_MFMA_LUT, 28672, 8192, 1, 7, 14, 1},   // 3-bit LUT 28672x8192 (two K groups)
    {wq::KIND_MFMA_LUT3D, 28672, 8192, 1, 8, 16, 1}, // 3-bit LUT 28672x8192, dense codes (two K groups)
    {wq::KIND_GEMV_FP8, 6144, 5120, 1, 2, 8, 1},     // attention Q (other GEMV shapes: the FP8 rows)
    {wq::KIND_GEMV_FP8, 1024, 5120, 1, 2, 8, 1},     // attention K, V
};

// Plans with K parts across work-groups, used when the caller passes a
// workspace.  Measured on MI355X (exactness-gated sweep over tilings and 1..8
// parts): the FFN down projection runs 19.7 us against 22.8 us in one part;
// for the attention shapes (K <= 6144) one part stays fastest, the second
// kernel's ~1.8 us outweighing the fuller grid.
constexpr TableEntry kSplitTable[] = {
    {wq::KIND_MFMA_FP8, 5120, 17408, 1, 5, 5, 4},    // FFN down
};

// The automatic rule splits K only while every part keeps this many K blocks.
constexpr int kMinPartBlocks = 32;

// ws: whether the call brings a workspace (K parts across work-groups allowed)
Plan make_plan(int kind, int64_t N, int64_t K, int cu, const Options& o, bool ws)
{
    Plan p;
    p.kind = kind;
    p.n_tiles = (int)(N / 16);
    p.KB = (int)(K / 128);
    ws = ws && kind != wq::KIND_GEMV_FP8;      // the GEMV keeps its K split inside the work-group
    // the W8A8 streaming tile streams the FP8 tile's units: it takes that tile's measured plans
    const int tkind = kind == wq::KIND_W8A8_STREAM ? wq::KIND_MFMA_FP8 : kind;
    const TableEntry* te = nullptr;
    if (cu == 256) {
        if (ws)
            for (const TableEntry& e : kSplitTable)
                if (e.kind == tkind && e.N == N && e.K == K) te = &e;
        if (!te)
            for (const TableEntry& e : kTable)
                if (e.kind == tkind && e.N == N && e.K == K) te = &e;
        // the GEMV streams the same one-tile units as the FP8 MFMA tile
        if (!te && kind == wq::KIND_GEMV_FP8)
            for (const TableEntry& e : kTable)
                if (e.kind == wq::KIND_MFMA_FP8 && e.N == N && e.K == K) te = &e;
    }
    const bool one_tile = kind == wq::KIND_GEMV_FP8 || kind == wq::KIND_W8A8_STREAM;
    if (o.nt || o.sn) {
        p.nt = one_tile ? 1 : (o.nt ? o.nt : 1);
        p.sn = o.sn ? std::min(o.sn, 8) : 1;
    } else if (te) {
        p.nt = one_tile ? 1 : te->nt;
        p.sn = te->sn;
    } else {
        // one tile per wave; as many column-waves per work-group as leaves at
        // least one work-group per compute unit (at most 8)
        p.nt = 1;
        p.sn = std::max(1, std::min(8, p.n_tiles / std::max(1, cu)));
    }
    const int group = p.nt * p.sn;
    p.n_cg = (p.n_tiles + group - 1) / group;
    // K parts: from the options or the table; otherwise, for a grid of at
    // most half the CUs and a long K, as many parts as bring it to about one
    // work-group per CU with kMinPartBlocks K blocks or more each.  Every
    // part keeps at least one aligned K block.
    const int kba = (p.KB + wq::k_align(kind) - 1) / wq::k_align(kind);
    int kp = 1;
    if (ws) {
        if (o.kp) kp = o.kp;
        else if (te && !o.nt && !o.sn) kp = te->kp;
        else if (2 * p.n_cg <= cu) kp = std::min(cu / p.n_cg, p.KB / kMinPartBlocks);
    }
    p.kp = std::max(1, std::min(kp, std::min(kba, wq::kMaxKParts)));
    int max_sk = std::min(wq::max_split(kind, p.nt, p.sn) / p.sn, kba / p.kp);   // every K group gets >= 1 block
    max_sk = std::min(max_sk, wq::kMaxKGroups);
    int sk;
    if (o.split) sk = std::max(1, o.split / p.sn);
    else if (te && !o.nt && !o.sn) sk = te->split / te->sn;
    else {
        // aim at `waves_per_cu` resident waves per compute unit
        const double target = (double)cu * o.waves_per_cu;
        sk = (int)std::lround(target / ((double)p.n_cg * p.kp * p.sn));
    }
    sk = std::max(1, std::min(sk, max_sk));
    p.split = sk * p.sn;
    return p;
}

// Workspace bytes of a plan: FP32 partials [kp][rows][N] for up to 32 rows
// per launch (0 when the plan has one K part).
size_t plan_workspace_bytes(const Plan& p, int64_t N) { return p.kp > 1 ? (size_t)p.kp * 32 * (size_t)N * 4 : 0; }

// Plans depend only on (kind, N, K, CU count, whether a workspace is given,
// options); cache them so the per-call host work is a lookup.
struct PlanKey {
    int kind;
    int64_t N, K;
    int cu;
    bool ws;
    bool operator==(const PlanKey& o) const
    {
        return kind == o.kind && N == o.N && K == o.K && cu == o.cu && ws == o.ws;
    }
};

constexpr int kPlanCache = 64;
std::mutex g_plan_mu;
PlanKey g_plan_keys[kPlanCache];
Plan g_plans[kPlanCache];
int g_plan_count = 0, g_plan_next = 0;

// Forgets the cached W8A8 call plans; the caller holds g_plan_mu.
void w8_cache_reset();

Plan cached_plan(int kind, int64_t N, int64_t K, int cu, bool ws)
{
    const PlanKey key{kind, N, K, cu, ws};
    options();   // read the environment once, before the first plan
    std::lock_guard<std::mutex> lk(g_plan_mu);
    for (int i = 0; i < g_plan_count; ++i)
        if (g_plan_keys[i] == key) return g_plans[i];
    Plan p = make_plan(kind, N, K, cu, g_opts, ws);
    g_plan_keys[g_plan_next] = key;
    g_plans[g_plan_next] = p;
    g_plan_next = (g_plan_next + 1) % kPlanCache;
    g_plan_count = std::min(g_plan_count + 1, kPlanCache);
    return p;
}

// Size limits keep every offset the kernels form within its width: a wave's
// run of tiles (at most 2 x 2^17 K blocks x 2 KiB) within a 32-bit buffer
// range, and the pack/unpack launches (one work-item per 16 or 32 codes)
// under 2^32 work-items.
constexpr int64_t kMaxDim = (int64_t)1 << 24;
constexpr int64_t kMaxCodes = (int64_t)1 << 35;

// Largest compute-unit count the plan queries accept.
constexpr int kMaxQueryCu = 1024;

bool shape_ok(int fmt, int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0 || K % 128) return false;
    if (N > kMaxDim || K > kMaxDim || N * K > kMaxCodes) return false;
    if (fmt == WQ_FMT_FP8_BLOCK) return N % 128 == 0;
    if (fmt == WQ_FMT_LUT3 || fmt == WQ_FMT_LUT3_DENSE) return N % 16 == 0;
    return false;
}

// Code bytes of a packed LUT matrix: 4 bits a code (nibbles) or 3 (dense).
size_t lut3_code_bytes(int fmt, int64_t N, int64_t K)
{
    return fmt == WQ_FMT_LUT3_DENSE ? (size_t)(N * K / 8 * 3) : (size_t)(N * K / 2);
}

// Group scales of the packed LUT matrix: per tile and run of 8 K blocks, 16
// rows x 8 FP16 (256 bytes); K block counts are padded to a multiple of 8.
size_t lut3_scale_bytes(int64_t N, int64_t K) { return (size_t)(N / 16) * (size_t)((K / 128 + 7) / 8) * 256; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The kernel family of a decode call: the LUT formats run their MFMA tile;
// FP8 runs the tile, or the GEMV for M <= 4 where the call or the
// WQ_FORCE_PATH lever asks for it (AUTO never does: kGemvAutoMaxM).
wq_status resolve_kind(int fmt, int path, int64_t M, int* kind)
{
    if (fmt != WQ_FMT_FP8_BLOCK) {
        if (path == WQ_PATH_GEMV) return WQ_ERR_PATH;
        *kind = fmt == WQ_FMT_LUT3_DENSE ? wq::KIND_MFMA_LUT3D : wq::KIND_MFMA_LUT;
        return WQ_OK;
    }
    int eff = path == WQ_PATH_AUTO ? options().force_path : path;
    if (eff == WQ_PATH_AUTO) eff = M <= kGemvAutoMaxM ? WQ_PATH_GEMV : WQ_PATH_MFMA;
    if (eff == WQ_PATH_GEMV && M > 4) {
        if (path == WQ_PATH_GEMV) return WQ_ERR_PATH;
        eff = WQ_PATH_MFMA;   // a forced GEMV lever only applies where it can run
    }
    *kind = eff == WQ_PATH_GEMV ? wq::KIND_GEMV_FP8 : wq::KIND_MFMA_FP8;
    return WQ_OK;
}

// Rows of x one launch serves.  One-tile MFMA waves serve M = 17..32 in one
// pass (each dequantised operand feeds both 16-row halves) -- for the LUT
// tile where its 32-row chunks fit; otherwise the rows 0..15 and 16..M-1 run
// as two passes.  Either way every row sees the same arithmetic as in a call
// of at most 16 rows.
int plan_rows_per_launch(const Plan& p)
{
    const bool single_pass =
        p.nt == 1 && (p.kind == wq::KIND_MFMA_FP8 || wq::lut_single_pass(p.kind, p.sn, p.split));
    return single_pass ? 32 : 16;
}

// Shared front end of the GEMMs.  static_scratch: the no-allocation entry
// point -- the workspace is the library's static device scratch of the
// current device (the caller passes none), planned as a call with a workspace.
wq_status gemm_common(int fmt, const void* packed, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                      uint16_t* y, int64_t ldy, int64_t M, void* workspace, size_t workspace_bytes, int path,
                      void* stream, bool static_scratch = false)
{
    // ---- validation that needs no HIP call
    if (M < 0 || M > 32) return WQ_ERR_SHAPE;
    if (!shape_ok(fmt, N, K)) return WQ_ERR_SHAPE;
    if (path != WQ_PATH_AUTO && path != WQ_PATH_GEMV && path != WQ_PATH_MFMA) return WQ_ERR_PATH;
    if (M == 0) return WQ_OK;
    if (!packed || !x || !y) return WQ_ERR_NULL;
    if (ldx < K || ldy < N) return WQ_ERR_LD;
    // the kernels address one launch's activations (up to 32 rows) with 32-bit byte offsets
    if (ldx > kMaxCodes || ((std::min<int64_t>(M, 32) - 1) * ldx + K) * 2 >= ((int64_t)1 << 32)) return WQ_ERR_LD;
    if (!aligned16(packed) || !aligned16(x) || ldx % 8) return WQ_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(y) & 1) return WQ_ERR_ALIGN;

    int kind;
    const wq_status ks = resolve_kind(fmt, path, M, &kind);
    if (ks != WQ_OK) return ks;

    // ---- device and workspace
    DevInfo dev;
    int dev_index = -1;
    wq_status st = current_device(&dev, &dev_index);
    if (st != WQ_OK) return st;
    const Plan p = cached_plan(kind, N, K, dev.cu, static_scratch || workspace != nullptr);
    if (static_scratch) {
        workspace = nullptr;
        workspace_bytes = 0;
        if (p.kp > 1) {
            if (plan_workspace_bytes(p, N) > wq::kScratchBytes) return WQ_ERR_SCRATCH;
            if (wq::scratch_address(dev_index, &workspace) != hipSuccess) return WQ_ERR_HIP;
            workspace_bytes = wq::kScratchBytes;
        }
    }
    if (p.kp > 1) {   // K parts across work-groups: FP32 partials in the workspace
        if (workspace_bytes < plan_workspace_bytes(p, N)) return WQ_ERR_WORKSPACE;
        if (!aligned16(workspace)) return WQ_ERR_ALIGN;
    }

    GemmArgs a{};
    const uint8_t* base = static_cast<const uint8_t*>(packed);
    a.codes = base;
    if (fmt == WQ_FMT_FP8_BLOCK) {
        a.scales = base + N * K;
        a.qmap = nullptr;
    } else {
        const size_t cb = lut3_code_bytes(fmt, N, K);
        a.scales = base + cb;
        a.qmap = reinterpret_cast<const uint16_t*>(base + cb + lut3_scale_bytes(N, K));
    }
    a.N = (int)N;
    a.KB = p.KB;
    a.n_tiles = p.n_tiles;
    a.n_cg = p.n_cg;
    a.sn = p.sn;
    a.kp = p.kp;
    a.ws = p.kp > 1 ? static_cast<float*>(workspace) : nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);

    const int64_t rows_per_launch = plan_rows_per_launch(p);
    for (int64_t r0 = 0; r0 < M; r0 += rows_per_launch) {
        const int rows = (int)std::min<int64_t>(rows_per_launch, M - r0);
        a.x = x + r0 * ldx;
        a.ldx = ldx;
        a.y = y + r0 * ldy;
        a.ldy = ldy;
        a.rows = rows;
        hipError_t e = wq::launch_gemm(kind, p.nt, kind == wq::KIND_GEMV_FP8 ? rows : 0, a, p.split, s);
        if (e != hipSuccess) return WQ_ERR_HIP;
    }
    return WQ_OK;
}

// Shared body of the two LUT packers (nibble and dense code layouts).
wq_status pack_lut3_common(int fmt, const uint8_t* codes, int64_t ldc, const uint16_t* qmap, const uint16_t* scales,
                           int64_t N, int64_t K, void* packed, void* hip_stream)
{
    if (!shape_ok(fmt, N, K)) return WQ_ERR_SHAPE;
    if (!codes || !qmap || !scales || !packed) return WQ_ERR_NULL;
    if (ldc < K) return WQ_ERR_LD;
    if (!aligned16(packed) || (reinterpret_cast<uintptr_t>(scales) & 1) || (reinterpret_cast<uintptr_t>(qmap) & 1))
        return WQ_ERR_ALIGN;
    DevInfo dev;
    wq_status st = current_device(&dev);
    if (st != WQ_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    uint8_t* pk = static_cast<uint8_t*>(packed);
    uint32_t* status = reinterpret_cast<uint32_t*>(pk + lut3_code_bytes(fmt, N, K) + lut3_scale_bytes(N, K) + 16);
    if (wq::launch_pack_lut3(codes, ldc, qmap, scales, N, K, pk, status, fmt == WQ_FMT_LUT3_DENSE, s) != hipSuccess)
        return WQ_ERR_HIP;
    uint32_t host_status = 0;
    if (hipMemcpyAsync(&host_status, status, sizeof(host_status), hipMemcpyDeviceToHost, s) != hipSuccess)
        return WQ_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return WQ_ERR_HIP;
    return host_status ? WQ_ERR_CODE : WQ_OK;
}

wq_status unpack_lut3_common(int fmt, const void* packed, int64_t N, int64_t K, uint16_t* w_f16, void* hip_stream)
{
    if (!shape_ok(fmt, N, K)) return WQ_ERR_SHAPE;
    if (!packed || !w_f16) return WQ_ERR_NULL;
    if (!aligned16(packed) || !aligned16(w_f16)) return WQ_ERR_ALIGN;
    DevInfo dev;
    wq_status st = current_device(&dev);
    if (st != WQ_OK) return st;
    return wq::launch_unpack_lut3(static_cast<const uint8_t*>(packed), N, K, w_f16, fmt == WQ_FMT_LUT3_DENSE,
                                  static_cast<hipStream_t>(hip_stream)) == hipSuccess
               ? WQ_OK
               : WQ_ERR_HIP;
}

}  // namespace

extern "C" {

const char* wq_status_str(wq_status s)
{
    switch (s) {
    case WQ_OK: return "WQ_OK";
    case WQ_ERR_NULL: return "WQ_ERR_NULL: required pointer is NULL";
    case WQ_ERR_SHAPE: return "WQ_ERR_SHAPE: unsupported M, N or K";
    case WQ_ERR_LD: return "WQ_ERR_LD: leading dimension smaller than the row";
    case WQ_ERR_WORKSPACE: return "WQ_ERR_WORKSPACE: workspace too small";
    case WQ_ERR_CODE: return "WQ_ERR_CODE: a 3-bit code exceeds 7";
    case WQ_ERR_DEVICE: return "WQ_ERR_DEVICE: current device is not gfx950";
    case WQ_ERR_HIP: return "WQ_ERR_HIP: HIP runtime call failed";
    case WQ_ERR_ALIGN: return "WQ_ERR_ALIGN: pointer or leading dimension misaligned";
    case WQ_ERR_PATH: return "WQ_ERR_PATH: path cannot serve this format or M";
    case WQ_ERR_SCRATCH: return "WQ_ERR_SCRATCH: the shape's K-split plan needs more than the static scratch";
    }
    return "WQ_ERR_UNKNOWN";
}

int wq_packed_format_version(void) { return kPackedFormatVersion; }

wq_status wq_set_tuning(int nt, int sn, int split, int waves_per_cu)
{
    if (nt < 0 || nt > 2 || sn < 0 || sn > 8) return WQ_ERR_SHAPE;
    if (split < 0 || split > 16 || waves_per_cu < 0 || waves_per_cu > 32) return WQ_ERR_SHAPE;
    options();
    std::lock_guard<std::mutex> lk(g_plan_mu);
    g_opts.nt = nt;
    g_opts.sn = sn;
    g_opts.split = split;
    g_opts.waves_per_cu = waves_per_cu ? waves_per_cu : 4;
    g_plan_count = 0;
    g_plan_next = 0;
    w8_cache_reset();
    return WQ_OK;
}

wq_status wq_set_kparts(int kp)
{
    if (kp < 0 || kp > wq::kMaxKParts) return WQ_ERR_SHAPE;
    options();
    std::lock_guard<std::mutex> lk(g_plan_mu);
    g_opts.kp = kp;
    g_plan_count = 0;
    g_plan_next = 0;
    w8_cache_reset();
    return WQ_OK;
}

wq_status wq_set_w8a8_stages(int stages)
{
    if (stages != 0 && stages != 2 && stages != 4) return WQ_ERR_SHAPE;
    options();
    std::lock_guard<std::mutex> lk(g_plan_mu);
    g_opts.w8a8_stages = stages;
    return WQ_OK;
}

size_t wq_fp8_block_packed_bytes(int64_t N, int64_t K)
{
    if (!shape_ok(WQ_FMT_FP8_BLOCK, N, K)) return 0;
    return (size_t)(N * K) + 4 * (size_t)(N / 128) * (size_t)(K / 128);
}

size_t wq_lut3_packed_bytes(int64_t N, int64_t K)
{
    if (!shape_ok(WQ_FMT_LUT3, N, K)) return 0;
    return lut3_code_bytes(WQ_FMT_LUT3, N, K) + lut3_scale_bytes(N, K) + 32;
}

size_t wq_lut3_dense_packed_bytes(int64_t N, int64_t K)
{
    if (!shape_ok(WQ_FMT_LUT3_DENSE, N, K)) return 0;
    return lut3_code_bytes(WQ_FMT_LUT3_DENSE, N, K) + lut3_scale_bytes(N, K) + 32;
}

wq_status wq_pack_fp8_block(const uint8_t* w_e4m3, int64_t ldw, const float* scales, int64_t N, int64_t K,
                            void* packed, void* hip_stream)
{
    if (!shape_ok(WQ_FMT_FP8_BLOCK, N, K)) return WQ_ERR_SHAPE;
    if (!w_e4m3 || !scales || !packed) return WQ_ERR_NULL;
    if (ldw < K) return WQ_ERR_LD;
    if (!aligned16(packed) || (reinterpret_cast<uintptr_t>(scales) & 3)) return WQ_ERR_ALIGN;
    DevInfo dev;
    wq_status st = current_device(&dev);
    if (st != WQ_OK) return st;
    hipError_t e = wq::launch_pack_fp8(w_e4m3, ldw, scales, N, K, static_cast<uint8_t*>(packed),
                                       static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? WQ_OK : WQ_ERR_HIP;
}

wq_status wq_gemm_fp8_block(const void* packed, int64_t N, int64_t K, const uint16_t* x, int64_t ldx, uint16_t* y,
                            int64_t ldy, int64_t M, void* workspace, size_t workspace_bytes, void* hip_stream)
{
    return gemm_common(WQ_FMT_FP8_BLOCK, packed, N, K, x, ldx, y, ldy, M, workspace, workspace_bytes,
                       WQ_PATH_AUTO, hip_stream);
}

wq_status wq_gemm_fp8_block_path(const void* packed, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                                 uint16_t* y, int64_t ldy, int64_t M, void* workspace, size_t workspace_bytes,
                                 int path, void* hip_stream)
{
    return gemm_common(WQ_FMT_FP8_BLOCK, packed, N, K, x, ldx, y, ldy, M, workspace, workspace_bytes, path,
                       hip_stream);
}

wq_status wq_gemm_fp8_block_noalloc(const void* packed, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                                    uint16_t* y, int64_t ldy, int64_t M, void* hip_stream)
{
    return gemm_common(WQ_FMT_FP8_BLOCK, packed, N, K, x, ldx, y, ldy, M, nullptr, 0, WQ_PATH_AUTO, hip_stream,
                       true);
}

size_t wq_noalloc_scratch_bytes(void) { return wq::kScratchBytes; }

wq_status wq_pack_lut3(const uint8_t* codes, int64_t ldc, const uint16_t* qmap, const uint16_t* scales, int64_t N,
                       int64_t K, void* packed, void* hip_stream)
{
    return pack_lut3_common(WQ_FMT_LUT3, codes, ldc, qmap, scales, N, K, packed, hip_stream);
}

wq_status wq_pack_lut3_dense(const uint8_t* codes, int64_t ldc, const uint16_t* qmap, const uint16_t* scales,
                             int64_t N, int64_t K, void* packed, void* hip_stream)
{
    return pack_lut3_common(WQ_FMT_LUT3_DENSE, codes, ldc, qmap, scales, N, K, packed, hip_stream);
}

wq_status wq_gemm_lut3(const void* packed, int64_t N, int64_t K, const uint16_t* x, int64_t ldx, uint16_t* y,
                       int64_t ldy, int64_t M, void* workspace, size_t workspace_bytes, void* hip_stream)
{
    return gemm_common(WQ_FMT_LUT3, packed, N, K, x, ldx, y, ldy, M, workspace, workspace_bytes, WQ_PATH_AUTO,
                       hip_stream);
}

wq_status wq_gemm_lut3_dense(const void* packed, int64_t N, int64_t K, const uint16_t* x, int64_t ldx, uint16_t* y,
                             int64_t ldy, int64_t M, void* workspace, size_t workspace_bytes, void* hip_stream)
{
    return gemm_common(WQ_FMT_LUT3_DENSE, packed, N, K, x, ldx, y, ldy, M, workspace, workspace_bytes,
                       WQ_PATH_AUTO, hip_stream);
}

size_t wq_gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K)
{
    // The plan with a workspace may split K across work-groups; its FP32
    // partials take kp * 32 * N * 4 bytes, for any M (rows per launch <= 32).
    (void)M;
    if (!shape_ok(fmt, N, K)) return 0;
    DevInfo dev;
    if (current_device(&dev) != WQ_OK) return 0;
    const int kind = fmt == WQ_FMT_FP8_BLOCK ? wq::KIND_MFMA_FP8
                     : fmt == WQ_FMT_LUT3_DENSE ? wq::KIND_MFMA_LUT3D
                                                : wq::KIND_MFMA_LUT;
    return plan_workspace_bytes(cached_plan(kind, N, K, dev.cu, true), N);
}

wq_status wq_query_gemm_plan(int fmt, int path, int64_t M, int64_t N, int64_t K, int cu, int with_workspace,
                             int* plan)
{
    if (!plan) return WQ_ERR_NULL;
    if (M < 1 || M > 32 || cu < 1 || cu > kMaxQueryCu || !shape_ok(fmt, N, K)) return WQ_ERR_SHAPE;
    if (path != WQ_PATH_AUTO && path != WQ_PATH_GEMV && path != WQ_PATH_MFMA) return WQ_ERR_PATH;
    int kind;
    const wq_status ks = resolve_kind(fmt, path, M, &kind);
    if (ks != WQ_OK) return ks;
    const Plan p = cached_plan(kind, N, K, cu, with_workspace != 0);
    const int rows = plan_rows_per_launch(p);
    plan[0] = kind == wq::KIND_GEMV_FP8 ? WQ_PATH_GEMV : WQ_PATH_MFMA;
    plan[1] = p.nt;
    plan[2] = p.sn;
    plan[3] = p.split;
    plan[4] = p.kp;
    plan[5] = (int)((M + rows - 1) / rows);
    return WQ_OK;
}

wq_status wq_unpack_fp8_block(const void* packed, int64_t N, int64_t K, uint16_t* w_bf16, void* hip_stream)
{
    if (!shape_ok(WQ_FMT_FP8_BLOCK, N, K)) return WQ_ERR_SHAPE;
    if (!packed || !w_bf16) return WQ_ERR_NULL;
    if (!aligned16(packed) || !aligned16(w_bf16)) return WQ_ERR_ALIGN;
    DevInfo dev;
    wq_status st = current_device(&dev);
    if (st != WQ_OK) return st;
    return wq::launch_unpack_fp8(static_cast<const uint8_t*>(packed), N, K, w_bf16, false,
                                 static_cast<hipStream_t>(hip_stream)) == hipSuccess
               ? WQ_OK
               : WQ_ERR_HIP;
}

wq_status wq_unpack_fp8_block_f32(const void* packed, int64_t N, int64_t K, float* w_f32, void* hip_stream)
{
    if (!shape_ok(WQ_FMT_FP8_BLOCK, N, K)) return WQ_ERR_SHAPE;
    if (!packed || !w_f32) return WQ_ERR_NULL;
    if (!aligned16(packed) || !aligned16(w_f32)) return WQ_ERR_ALIGN;
    DevInfo dev;
    wq_status st = current_device(&dev);
    if (st != WQ_OK) return st;
    return wq::launch_unpack_fp8(static_cast<const uint8_t*>(packed), N, K, w_f32, true,
                                 static_cast<hipStream_t>(hip_stream)) == hipSuccess
               ? WQ_OK
               : WQ_ERR_HIP;
}

wq_status wq_unpack_lut3(const void* packed, int64_t N, int64_t K, uint16_t* w_f16, void* hip_stream)
{
    return unpack_lut3_common(WQ_FMT_LUT3, packed, N, K, w_f16, hip_stream);
}

wq_status wq_unpack_lut3_dense(const void* packed, int64_t N, int64_t K, uint16_t* w_f16, void* hip_stream)
{
    return unpack_lut3_common(WQ_FMT_LUT3_DENSE, packed, N, K, w_f16, hip_stream);
}

// ------------------------------------------------------------------ W8A8

}  // extern "C"

namespace {

// K blocks per W8A8 K part of the automatic rule for grids of more than one
// 128 x 128 tile per CU, and the fewest K blocks a part keeps for smaller ones.
constexpr int kW8PartBlocks = 40;
constexpr int kW8MinPartBlocks = 12;

struct W8Plan {
    int tile;   // wq::W8Tile
    int kp;     // K parts across work-groups
};

// Estimated microseconds of a GEMM on 128 x 128 or 256 x 256 tiles, for the
// choice between them at 256 < Mpad <= kW8BigM.  Per K block of a part: a
// round of 128 x 128 work-groups at two per CU takes ~1.07 us, one at one per
// CU (the four-stage pipeline) ~0.75 us, a round of 256 x 256 work-groups
// (one per CU) ~1.75 us; a 128 x 128 grid of several rounds adds ~20 us, and
// a partial last round costs at least half a round.  K parts add their FP32
// partials written and read back (~6 TB/s) and the summing kernel (~3 us).
// Fitted to the FFN shapes at M = 192 ... 8192 (gate/up K = 5120 and down
// K = 17408, 1-6 K parts, both tiles); on those the estimate ranks the two
// tiles as measured wherever they differ by more than 3%.
double w8_estimate_us(int tile, int64_t tiles, int kp, int KB, int64_t M, int64_t N, int cu)
{
    const int64_t n = tiles * kp;
    const double bpp = (double)((KB + kp - 1) / kp);
    double t;
    if (tile == wq::W8_T128) {
        if (n <= cu) t = 0.754 * bpp;
        else {
            const double r = (double)n / (2.0 * cu);
            t = 20.0 + 1.07 * bpp * std::max(r, std::ceil(r) - 0.5);
        }
    } else t = std::ceil((double)n / cu) * 1.75 * bpp;
    if (kp > 1) t += 2.0 * kp * (double)M * (double)N * 4.0 / 6.0e6 + 3.0;
    return t;
}

// WQ_W8A8_TILE = 128 | 256 | 64 (64 x 128) | 6464 (64 x 64): one tile for
// every M (sweeps); read once.
int forced_w8a8_tile()
{
    static const int t = [] {
        const char* p = std::getenv("WQ_W8A8_TILE");
        const int v = p ? std::atoi(p) : 0;
        return v == 128 ? wq::W8_T128 : v == 256 ? wq::W8_T256 : v == 64 ? wq::W8_T64x128
                                                   : v == 6464 ? wq::W8_T64x64 : -1;
    }();
    return t;
}

// Tile and K parts of a W8A8 call (ws: the call brings a workspace, so K may
// be split across work-groups; the wq_set_kparts value forces the count):
// - the tile: 64 x 128 or 64 x 64 for Mpad <= 64, 128 x 128 up to kW8BigM
//   rows, 256 x 256 above (see the launcher);
// - where the grid has at most one tile per CU, or the tile has 64 rows:
//   among the candidate tiles and part counts (each part keeping at least
//   kW8MinPartBlocks K blocks), the pair that best fills the work-group slots
//   -- one per CU for a grid the four-stage pipeline runs, two per CU for the
//   two-stage one; a pair must fill 5% more slots than the best so far, or
//   as many with fewer parts (with more parts above 128 rows), and ties go
//   to the larger tile.  Measured on
//   MI355X (GEMM + parts sum, M = 16 / 32 / 48 / 64, quantised activations
//   prepared): FFN down takes 64 x 64 in 3 parts, 21.9 / 22.4 / 22.9 /
//   23.9 us (128 x 128 in 6 parts: 25.9 / 26.6 / 27.7 / 29.4; in one part
//   ~100); gate/up takes 64 x 128 in 3 parts, 22.2 / 23.5 / 25.7 / 27.5 us
//   (128 x 128 in 3 parts: 23.3 / 25.2 / 27.1 / 29.5).  At M = 96 / 128 the
//   128 x 128 tile: down 6 parts 30.8 / 32.9 us, gate/up 3 parts 33.0 /
//   36.5.  FFN down at M = 192 / 256 (80 tiles): 6 parts, two work-groups
//   per CU, 38.0 / 45.5 us against 45.0 / 46.4 in 3 with one per CU;
// - a 128 x 128 grid of 1 to 4 tiles per CU: one part per kW8PartBlocks K
//   blocks, but no more parts than bring the grid to 4 work-groups per CU.
//   Measured: FFN down at M = 512 / 1024 / 2048 runs 118 / 143 / 239 us in
//   one part and 74 / 124 / 224 us in 3, 3 and 2 parts;
//   gate/up (K = 5120) is fastest in one part from M = 256 on;
// - at 256 < Mpad <= kW8BigM and K >= 4096 the 256 x 256 tile replaces
//   that plan where w8_estimate_us puts it 5% lower (its fewer, larger
//   work-groups do more matrix-core work per byte staged, but fill the CUs
//   in coarser rounds).  Measured against the 128 x 128 plan (same process,
//   interleaved): gate/up M = 512 / 768 / 1500 / 2500 / 3500 / 4096 in one
//   part 72.9 / 77.0 / 146.6 / 228.8 / 309.3 / 372.2 us against 81.0 /
//   91.8 / 165.3 / 253.8 / 346.1 / 393.0; FFN down M = 800 / 1024 / 1200 /
//   2048 / 3000 in 3, 3, 2, 3 and 1 parts 93.5 / 104.2 / 123.6 / 198.8 /
//   246.6 against 109.3 / 126.2 / 157.0 / 226.8 / 316.5; where the 128 x 128
//   plan stays (gate/up M = 300 / 800 / 1024 / 2048, down M = 300 ... 768
//   and 3500 / 4096) the two are within 2.5%;
// - above kW8BigM the 256 x 256 tile, with K whole.
W8Plan w8a8_plan(int64_t M, int64_t N, int64_t K, int cu, bool ws)
{
    int forced_kp;
    {
        std::lock_guard<std::mutex> lk(g_plan_mu);
        forced_kp = g_opts.kp;
    }
    const int KB = (int)(K / 128);
    const int max_kp = std::max(1, std::min(KB, wq::kMaxKParts));
    const int64_t mpad = (M + 15) / 16 * 16;
    // Up to 64 rows the product runs on the weight-streaming tile with the FP8
    // decode tile's plan for the shape (unless a tile is forced), while each
    // work-group's staged activations (Mpad x K codes) are at most twice its
    // weight bytes (16 sn x K): measured against the 64-row tiles (GEMM and
    // parts sum, quantised activations prepared), gate/up M = 1 / 16 / 32 /
    // 48 / 64 16.3 / 16.5 / 17.4 / 19.9 / 20.2 us against 20.6 / 21.5 /
    // 23.1 / 25.0 / 26.7; FFN down (4 parts) 18.4 / 18.9 / 19.9 / 22.0 /
    // 23.1 against 21.0 / 21.6 / 22.1 / 22.5 / 23.2; attention Q 8.5 / 8.7 /
    // 10.0 / 12.6 / 13.0 against 11.6 / 12.0 / 12.6 / 12.9 / 13.1; attention
    // K/V (one column-wave a work-group) 5.7 / 6.0 / 7.4 at M <= 32 against
    // 8.6 / 9.2 / 9.7, but 10.8 / 11.0 at M = 48 / 64 against 9.8 -- there
    // every work-group stages four times its weight bytes.
    if (mpad <= 64 && forced_w8a8_tile() < 0) {
        const Plan sp = cached_plan(wq::KIND_W8A8_STREAM, N, K, cu, ws);
        if (mpad <= 32 * sp.sn) return {wq::W8_STREAM, sp.kp};
    }
    int cand[2], nc = 0;
    if (forced_w8a8_tile() >= 0) cand[nc++] = forced_w8a8_tile();
    else if (mpad <= 64) {
        cand[nc++] = wq::W8_T64x128;
        cand[nc++] = wq::W8_T64x64;
    } else cand[nc++] = mpad > wq::kW8BigM ? wq::W8_T256 : wq::W8_T128;
    auto tiles = [&](int t) {
        const int r = wq::w8_tile_rows(t), c = wq::w8_tile_cols(t);
        return (mpad + r - 1) / r * ((N + c - 1) / c);
    };
    auto fill = [&](int64_t n) {   // share of the work-group slots a grid of n fills
        return n <= cu ? (double)n / cu : n <= 2 * (int64_t)cu ? (double)n / (2.0 * cu) : 0.0;
    };
    // 256 < Mpad <= kW8BigM and K >= 4096 (the range the estimate was fitted
    // on): the 256 x 256 tile instead of a 128 x 128 plan where its estimate
    // is at least 5% lower -- in one K part, or in up to three (each of
    // kW8MinPartBlocks K blocks or more) for a grid of fewer tiles than CUs; a
    // forced part count is kept
    auto big_tile_if_faster = [&](W8Plan p) {
        if (p.tile != wq::W8_T128 || mpad <= 256 || KB < 32 || forced_w8a8_tile() >= 0) return p;
        const int64_t t256 = tiles(wq::W8_T256);
        W8Plan b = p;
        double bt = 0.95 * w8_estimate_us(wq::W8_T128, tiles(wq::W8_T128), p.kp, KB, M, N, cu);
        const bool fixed_kp = forced_kp || !ws;
        const int kmin = fixed_kp ? p.kp : 1;
        const int kmax = fixed_kp ? p.kp
                         : t256 < cu ? std::min(3, std::max(1, std::min(max_kp, KB / kW8MinPartBlocks)))
                                     : 1;
        for (int k = kmin; k <= kmax; ++k) {
            const double e = w8_estimate_us(wq::W8_T256, t256, k, KB, M, N, cu);
            if (e < bt) {
                bt = e;
                b = {wq::W8_T256, k};
            }
        }
        return b;
    };
    W8Plan best{cand[0], 1};
    if (!ws || forced_kp) {                          // the part count is given: the tile that fills best
        const int kp = ws ? std::min(forced_kp, max_kp) : 1;
        double bf = -1.0;
        for (int i = 0; i < nc; ++i) {
            const int64_t n = tiles(cand[i]) * kp;
            const double f = n <= 2 * (int64_t)cu ? fill(n) : 1.0;
            if (f > bf + 1e-9) {
                bf = f;
                best = {cand[i], kp};
            }
        }
        return big_tile_if_faster(best);
    }
    if (cand[0] == wq::W8_T256) return best;
    const int64_t t0 = tiles(cand[0]);
    if (cand[0] == wq::W8_T128 && t0 > cu) {         // 1 to 4 tiles per CU
        if (t0 < 4 * (int64_t)cu)
            best.kp = std::max(1, (int)std::min<int64_t>({(int64_t)KB / kW8PartBlocks, (4 * cu + t0 - 1) / t0,
                                                          (int64_t)max_kp}));
        return big_tile_if_faster(best);
    }
    // equal fills: fewer parts while the tile has at most 128 rows (the
    // stream binds); more work-groups above (two per CU hide the longer
    // matrix-core work of each block)
    const bool more_wgs = mpad > 128;
    double bf = fill(t0);
    for (int i = 0; i < nc; ++i) {
        const int64_t nt = tiles(cand[i]);
        for (int k = 1; k <= std::min(max_kp, std::max(1, KB / kW8MinPartBlocks)); ++k) {
            const int64_t n = nt * k;
            if (n > 2 * (int64_t)cu) break;
            const double f = fill(n);
            if (f > bf + 0.05 || (f >= bf - 0.05 && (more_wgs ? k > best.kp : k < best.kp))) {
                bf = std::max(bf, f);
                best = {cand[i], k};
            }
        }
    }
    return big_tile_if_faster(best);
}

size_t w8a8_workspace_bytes(int64_t M, int64_t N, int kp) { return kp > 1 ? (size_t)kp * M * N * 4 : 0; }

// Work-group slots of one round of a tile-kernel grid of n work-groups:
// 256 x 256 tiles run one per CU, 128 x 128 tiles two per CU once the grid has
// more work-groups than CUs (the two-stage pipeline), else one.
int64_t w8_round_slots(int tile, int64_t n, int cu)
{
    return tile == wq::W8_T128 && n > cu ? 2 * (int64_t)cu : (int64_t)cu;
}

// Work-groups of a tile-kernel grid over M rows and N columns.
int64_t w8_grid(const W8Plan& p, int64_t M, int64_t N)
{
    const int64_t mpad = (M + 15) / 16 * 16;
    const int r = wq::w8_tile_rows(p.tile), c = wq::w8_tile_cols(p.tile);
    return (mpad + r - 1) / r * ((N + c - 1) / c) * p.kp;
}

// A W8A8 call: output columns [0, na) on `main`, and where na < N the columns
// [na, N) as a second launch on `tail`, the plan of that band as a call of
// its own.
struct W8Call {
    W8Plan main;
    int64_t na;
    W8Plan tail;
};

// Column bands.  A grid of several rounds of work-group slots whose last
// round is at most half full leaves most CUs idle for that round.  For
// 64 < Mpad <= kW8BigM, K >= 4096 (the range w8_estimate_us was fitted on)
// and no forced tile or part count, such a call is split by columns: the
// widest leading band -- a multiple of 256 columns, leaving at most a quarter
// of N -- whose own plan runs in one K part and fills whole rounds takes that
// plan, and the remaining columns run as a second launch with their own plan
// (with a workspace, K split over the slots), where the estimates of the two
// launches (plus ~3 us for the second) come to at least 5% below that of the
// one-band plan.  Each output is computed by one of the two launches; in the
// first band in one K part, the same sums as any one-part tile plan (without
// a workspace both bands keep K whole: the same bits as one band).  Measured
// on MI355X (quantised activations prepared, graph-replayed calls, the same
// process), with a workspace: gate/up M = 1024 / 2048 / 3000 / 4096
// 101.8 / 184.6 / 272.7 / 357.0 us against 122.2 / 207.2 / 288.7 / 368.8
// in one band, FFN down M = 4096 331.7 against 377.6, attention output
// M = 4096 135.1 against 138.8; without one: gate/up 113.5 / 189.9 / 272.2
// / 354.6 against 121.3 / 208.4 / 289.7 / 372.1, down M = 4096 355.1
// against 384.1, attention output 131.9 against 141.7.  Where the estimate
// keeps one band the split measured slower: FFN down without a workspace at
// M = 1921 / 2048 (the rest of the columns a whole extra round of 136 K
// blocks on half the CUs) 243.3 / 246.4 against 234.7 / 227.5; gate/up
// M = 512 (one partial round) 75.0 against 72.7; above kW8BigM, whose plans
// keep K whole, gate/up M = 5000 / 6144 / 8192 457.7 / 536.0 / 690.1
// against 442.6 / 519.5 / 675.2, FFN down M = 8192 676.3 against 664.5.
W8Call w8a8_call_uncached(int64_t M, int64_t N, int64_t K, int cu, bool ws)
{
    const W8Plan p = w8a8_plan(M, N, K, cu, ws);
    const W8Call one{p, N, W8Plan{p.tile, 1}};
    int forced_kp;
    {
        std::lock_guard<std::mutex> lk(g_plan_mu);
        forced_kp = g_opts.kp;
    }
    const int64_t mpad = (M + 15) / 16 * 16;
    const int KB = (int)(K / 128);
    if (forced_kp || forced_w8a8_tile() >= 0 || mpad > wq::kW8BigM || KB < 32 ||
        (p.tile != wq::W8_T128 && p.tile != wq::W8_T256))
        return one;
    const int64_t n = w8_grid(p, M, N), slots = w8_round_slots(p.tile, n, cu), last = n % slots;
    if (n <= slots || last == 0 || 2 * last > slots) return one;
    for (int64_t na = (N - 1) / 256 * 256; na >= 256 && 4 * (N - na) <= N; na -= 256) {
        const W8Plan pm = w8a8_plan(M, na, K, cu, ws);
        if (pm.kp != 1 || (pm.tile != wq::W8_T128 && pm.tile != wq::W8_T256)) continue;
        const int64_t nm = w8_grid(pm, M, na);
        if (nm % w8_round_slots(pm.tile, nm, cu)) continue;
        const W8Plan pt = w8a8_plan(M, N - na, K, cu, ws);
        const double two = w8_estimate_us(pm.tile, nm, 1, KB, M, na, cu) +
                           w8_estimate_us(pt.tile, w8_grid(pt, M, N - na) / pt.kp, pt.kp, KB, M, N - na, cu) + 3.0;
        if (two < 0.95 * w8_estimate_us(p.tile, n / p.kp, p.kp, KB, M, N, cu)) return {pm, na, pt};
        return one;
    }
    return one;
}

struct W8Key {
    int64_t M, N, K;
    int cu;
    bool ws;
    bool operator==(const W8Key& o) const { return M == o.M && N == o.N && K == o.K && cu == o.cu && ws == o.ws; }
};

constexpr int kW8Cache = 64;
W8Key g_w8_keys[kW8Cache];
W8Call g_w8_calls[kW8Cache];
int g_w8_count = 0, g_w8_next = 0;

void w8_cache_reset()
{
    g_w8_count = 0;
    g_w8_next = 0;
}

W8Call w8a8_call(int64_t M, int64_t N, int64_t K, int cu, bool ws)
{
    const W8Key key{M, N, K, cu, ws};
    options();   // read the environment once, before the first plan
    {
        std::lock_guard<std::mutex> lk(g_plan_mu);
        for (int i = 0; i < g_w8_count; ++i)
            if (g_w8_keys[i] == key) return g_w8_calls[i];
    }
    const W8Call c = w8a8_call_uncached(M, N, K, cu, ws);
    std::lock_guard<std::mutex> lk(g_plan_mu);
    g_w8_keys[g_w8_next] = key;
    g_w8_calls[g_w8_next] = c;
    g_w8_next = (g_w8_next + 1) % kW8Cache;
    g_w8_count = std::min(g_w8_count + 1, kW8Cache);
    return c;
}

size_t w8a8_call_workspace_bytes(const W8Call& c, int64_t M, int64_t N)
{
    const size_t a = w8a8_workspace_bytes(M, c.na, c.main.kp);
    const size_t b = c.na < N ? w8a8_workspace_bytes(M, N - c.na, c.tail.kp) : 0;
    return std::max(a, b);
}

}  // namespace

extern "C" {

size_t wq_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || !shape_ok(WQ_FMT_FP8_BLOCK, N, K) || !wq_x_fp8_packed_bytes(M, K)) return 0;
    DevInfo dev;
    if (current_device(&dev) != WQ_OK) return 0;
    return w8a8_call_workspace_bytes(w8a8_call(M, N, K, dev.cu, true), M, N);
}

wq_status wq_query_w8a8_plan(int64_t M, int64_t N, int64_t K, int cu, int with_workspace, int* plan)
{
    if (!plan) return WQ_ERR_NULL;
    if (M < 1 || cu < 1 || cu > kMaxQueryCu || !shape_ok(WQ_FMT_FP8_BLOCK, N, K) ||
        (uint64_t)N * (uint64_t)K >= ((uint64_t)1 << 32) || !wq_x_fp8_packed_bytes(M, K))
        return WQ_ERR_SHAPE;
    const W8Call c = w8a8_call(M, N, K, cu, with_workspace != 0);
    const W8Plan p = c.main;
    if (p.tile == wq::W8_STREAM) {   // rows of the row tiles, columns of a work-group
        const int64_t mpad = (M + 15) / 16 * 16;
        plan[0] = mpad <= 16 ? 16 : mpad <= 32 ? 32 : 64;
        plan[1] = 16 * cached_plan(wq::KIND_W8A8_STREAM, N, K, cu, with_workspace != 0).sn;
    } else {
        plan[0] = wq::w8_tile_rows(p.tile);
        plan[1] = wq::w8_tile_cols(p.tile);
    }
    plan[2] = p.kp;
    plan[3] = p.tile == wq::W8_STREAM ? 1 : 0;
    plan[4] = (int)c.na;
    plan[5] = c.na < N ? wq::w8_tile_rows(c.tail.tile) : 0;
    plan[6] = c.na < N ? wq::w8_tile_cols(c.tail.tile) : 0;
    plan[7] = c.na < N ? c.tail.kp : 0;
    return WQ_OK;
}

size_t wq_x_fp8_packed_bytes(int64_t M, int64_t K)
{
    if (M <= 0 || K <= 0 || K % 128 || M > (int64_t)1 << 24 || K > (int64_t)1 << 24) return 0;
    const int64_t mpad = (M + 15) / 16 * 16;
    const int64_t bytes = mpad * K + 4 * mpad * (K / 128);
    return bytes < ((int64_t)1 << 31) ? (size_t)bytes : 0;
}

wq_status wq_quantize_x_fp8(const uint16_t* x_bf16, int64_t ldx, int64_t M, int64_t K, void* xq, void* hip_stream)
{
    if (M < 0) return WQ_ERR_SHAPE;
    if (M == 0) return WQ_OK;
    if (!wq_x_fp8_packed_bytes(M, K)) return WQ_ERR_SHAPE;
    if (!x_bf16 || !xq) return WQ_ERR_NULL;
    if (ldx < K) return WQ_ERR_LD;
    if (!aligned16(x_bf16) || ldx % 8 || !aligned16(xq)) return WQ_ERR_ALIGN;
    DevInfo dev;
    wq_status st = current_device(&dev);
    if (st != WQ_OK) return st;
    return wq::launch_quantize_x(x_bf16, ldx, (int)M, (int)K, static_cast<uint8_t*>(xq),
                                 static_cast<hipStream_t>(hip_stream)) == hipSuccess
               ? WQ_OK
               : WQ_ERR_HIP;
}

wq_status wq_gemm_fp8_w8a8(const void* packed, int64_t N, int64_t K, const void* xq, int64_t M, uint16_t* y,
                           int64_t ldy, void* workspace, size_t workspace_bytes, void* hip_stream)
{
    if (M < 0) return WQ_ERR_SHAPE;
    if (!shape_ok(WQ_FMT_FP8_BLOCK, N, K) || (uint64_t)N * (uint64_t)K >= ((uint64_t)1 << 32)) return WQ_ERR_SHAPE;
    if (M == 0) return WQ_OK;
    if (!wq_x_fp8_packed_bytes(M, K)) return WQ_ERR_SHAPE;
    if (!packed || !xq || !y) return WQ_ERR_NULL;
    if (ldy < N) return WQ_ERR_LD;
    if (!aligned16(packed) || !aligned16(xq) || (reinterpret_cast<uintptr_t>(y) & 1)) return WQ_ERR_ALIGN;
    DevInfo dev;
    wq_status st = current_device(&dev);
    if (st != WQ_OK) return st;
    // with a workspace, K may be split across work-groups (FP32 partials there)
    const W8Call call = w8a8_call(M, N, K, dev.cu, workspace != nullptr);
    const W8Plan plan = call.main;
    const int kp = plan.kp;
    int stages;
    {
        std::lock_guard<std::mutex> lk(g_plan_mu);
        stages = g_opts.w8a8_stages;
    }
    if (const size_t need = w8a8_call_workspace_bytes(call, M, N)) {
        if (workspace_bytes < need) return WQ_ERR_WORKSPACE;
        if (!aligned16(workspace)) return WQ_ERR_ALIGN;
    }
    if (plan.tile == wq::W8_STREAM) {
        const Plan p = cached_plan(wq::KIND_W8A8_STREAM, N, K, dev.cu, workspace != nullptr);
        wq::GemmArgs a{};
        a.codes = static_cast<const uint8_t*>(packed);
        a.scales = static_cast<const uint8_t*>(packed) + N * K;
        a.qmap = nullptr;
        a.x = static_cast<const uint16_t*>(xq);
        a.ldx = (M + 15) / 16 * 16;
        a.y = y;
        a.ldy = ldy;
        a.rows = (int)M;
        a.N = (int)N;
        a.KB = p.KB;
        a.n_tiles = p.n_tiles;
        a.n_cg = p.n_cg;
        a.sn = p.sn;
        a.kp = p.kp;
        a.ws = p.kp > 1 ? static_cast<float*>(workspace) : nullptr;
        return wq::launch_gemm(wq::KIND_W8A8_STREAM, 1, 0, a, p.split, static_cast<hipStream_t>(hip_stream)) ==
                       hipSuccess
                   ? WQ_OK
                   : WQ_ERR_HIP;
    }
    // the packed matrix: 16 x K code bytes per 16-column tile, then the block
    // scales [N/128][K/128]; a band of columns starts at its first tile and
    // its first scale row
    const uint8_t* codes = static_cast<const uint8_t*>(packed);
    const float* sw = reinterpret_cast<const float*>(codes + N * K);
    const uint8_t* xqb = static_cast<const uint8_t*>(xq);
    float* ws = static_cast<float*>(workspace);
    const hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = wq::launch_w8a8(codes, sw, (int)call.na, (int)K, xqb, (int)M, y, ldy, plan.tile, kp,
                                   kp > 1 ? ws : nullptr, dev.cu, stages, s);
    if (e == hipSuccess && call.na < N) {
        const int tkp = call.tail.kp;
        e = wq::launch_w8a8(codes + call.na * K, sw + call.na / 128 * (K / 128), (int)(N - call.na), (int)K, xqb,
                            (int)M, y + call.na, ldy, call.tail.tile, tkp, tkp > 1 ? ws : nullptr, dev.cu, stages, s);
    }
    return e == hipSuccess ? WQ_OK : WQ_ERR_HIP;
}

wq_status wq_unpack_x_fp8(const void* xq, int64_t M, int64_t K, uint8_t* codes, float* scales, void* hip_stream)
{
    if (M < 0) return WQ_ERR_SHAPE;
    if (M == 0) return WQ_OK;
    if (!wq_x_fp8_packed_bytes(M, K)) return WQ_ERR_SHAPE;
    if (!xq || !codes || !scales) return WQ_ERR_NULL;
    if (!aligned16(xq) || (reinterpret_cast<uintptr_t>(scales) & 3)) return WQ_ERR_ALIGN;
    DevInfo dev;
    wq_status st = current_device(&dev);
    if (st != WQ_OK) return st;
    return wq::launch_unpack_x(static_cast<const uint8_t*>(xq), (int)M, (int)K, codes, scales,
                               static_cast<hipStream_t>(hip_stream)) == hipSuccess
               ? WQ_OK
               : WQ_ERR_HIP;
}

}  // extern "C"
