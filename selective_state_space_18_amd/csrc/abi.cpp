// libssmscan C ABI: argument validation, work planning, scratch memory and
// kernel dispatch.  Every argument check runs before the first HIP call, so
// argument errors enqueue nothing and need no device.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "ssm_launch.h"
#include "ssmscan.h"

namespace {

constexpr int kVersion = 10000;   // 1.0.0
constexpr int kWavesPerBlock = 4;  // scan blocks: 4 independent 64-channel waves
constexpr int64_t kMinSegment = 64;
// Scan blocks per CU the planner aims for.  The structured kernels hold about
// ten 4-wave blocks per CU at once; more blocks than that keep every SIMD fed
// while the last ones drain, at the price of a longer carry pass.
constexpr int64_t kBlocksPerCu = 16;

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return SSM_OK;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(SSM_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

std::atomic<int64_t> g_opt_segment_len{0};
std::atomic<int64_t> g_opt_force_general{0};
std::atomic<int64_t> g_opt_profile{0};
std::atomic<int64_t> g_opt_step_channels{4};

// ---------------------------------------------------------------------------
// Optional per-kernel event timing (SSM_OPT_PROFILE).

struct ProfRec {
    hipEvent_t a, b;
    int kind;
};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof;

template <typename F>
hipError_t timed(int kind, hipStream_t s, F launch) {
    if (!g_opt_profile.load()) return launch();
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    if (e == hipSuccess) e = hipEventRecord(a, s);
    if (e != hipSuccess) {
        if (a) (void)hipEventDestroy(a);
        if (b) (void)hipEventDestroy(b);
        return e;
    }
    hipError_t le = launch();
    e = hipEventRecord(b, s);
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        g_prof.push_back({a, b, kind});
    }
    return le != hipSuccess ? le : e;
}

bool supported_n(int64_t N) { return N == 1 || N == 2 || N == 4 || N == 8 || N == 16; }

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// A tensor argument: pointer, element count, element size, name.
struct Arg {
    const void *p;
    int64_t count;
    int64_t esize;
    const char *name;
    uintptr_t lo() const { return reinterpret_cast<uintptr_t>(p); }
    uintptr_t hi() const { return lo() + (uintptr_t)(count * esize); }
};

int check_args(const Arg *args, int n) {
    for (int i = 0; i < n; ++i) {
        const Arg &a = args[i];
        int64_t bytes;
        if (!mul_ok(a.count, a.esize, &bytes) || bytes > (INT64_MAX >> 2))
            return fail(SSM_ERR_BAD_DIM, "%s: size overflows", a.name);
        if (a.count > 0 && a.p == nullptr)
            return fail(SSM_ERR_NULLPTR, "%s is NULL but has %lld elements", a.name, (long long)a.count);
        if (a.p != nullptr && (a.lo() % (uintptr_t)a.esize) != 0)
            return fail(SSM_ERR_ALIGN, "%s (%p) is not aligned to its %lld-byte element", a.name, a.p,
                        (long long)a.esize);
    }
    return SSM_OK;
}

bool overlaps(const Arg &a, const Arg &b) {
    if (a.count == 0 || b.count == 0 || a.p == nullptr || b.p == nullptr) return false;
    return a.lo() < b.hi() && b.lo() < a.hi();
}

int check_output(const Arg &out, const Arg *others, int n) {
    for (int i = 0; i < n; ++i)
        if (overlaps(out, others[i]))
            return fail(SSM_ERR_ALIAS, "%s overlaps %s", out.name, others[i].name);
    return SSM_OK;
}

int64_t dtype_size(int dtype) { return dtype == SSM_F32 ? 4 : 2; }

// ---------------------------------------------------------------------------
// Planning

struct Plan {
    int S;
    int64_t seg_len;
    int tiles_per_b;
    int n_tiles;
};

// Time segments: enough 4-wave blocks to give every CU an equal whole number
// (>= kBlocksPerCu) of them when that is possible, with segments of at least kMinSegment
// steps.  Channels are never split; only time is.  A segment never spans more
// than 1 GiB of x (the kernels address it with 32-bit buffer offsets) and the
// grid stays below 2^30 blocks.
Plan make_plan(int64_t Bsz, int64_t L, int64_t Dm, int64_t esize, int cus) {
    Plan pl;
    pl.tiles_per_b = (int)((Dm + 63) / 64);
    pl.n_tiles = (int)(Bsz * pl.tiles_per_b);
    const int64_t bps = (pl.n_tiles + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t row = (Dm > 0 ? Dm : 1) * esize;
    const int64_t max_len = ((int64_t)1 << 30) / row > 1 ? ((int64_t)1 << 30) / row : 1;
    int64_t S = 1;
    const int64_t forced = g_opt_segment_len.load();
    if (L <= 0 || bps == 0) {
        S = 1;
    } else if (forced > 0) {
        const int64_t max_seg = ((int64_t)1 << 30) / (bps > 0 ? bps : 1);
        int64_t sl = forced < L ? forced : L;
        if (sl > max_len) sl = max_len;
        if ((L + sl - 1) / sl > max_seg) sl = (L + max_seg - 1) / max_seg;
        pl.seg_len = sl;
        pl.S = (int)((L + sl - 1) / sl);
        return pl;
    } else {
        const int64_t cap = L / kMinSegment > 1 ? L / kMinSegment : 1;
        const int64_t c = cus > 0 ? cus : 256;
        S = (kBlocksPerCu * c + bps - 1) / bps;  // fallback: at least kBlocksPerCu per CU
        for (int64_t m = kBlocksPerCu; m <= kBlocksPerCu + kBlocksPerCu / 2; ++m) {
            if ((m * c) % bps == 0) {
                S = m * c / bps;
                break;
            }
        }
        if (S > cap) S = cap;
        if (S < 1) S = 1;
        if ((L + S - 1) / S > max_len) S = (L + max_len - 1) / max_len;
    }
    pl.seg_len = L > 0 ? (L + S - 1) / S : 1;
    pl.S = L > 0 ? (int)((L + pl.seg_len - 1) / pl.seg_len) : 1;
    return pl;
}

std::mutex g_dev_mu;
std::map<int, int> g_cus;

int device_cus(int dev, int *cus) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    auto it = g_cus.find(dev);
    if (it != g_cus.end()) {
        *cus = it->second;
        return SSM_OK;
    }
    int v = 0;
    hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
    g_cus[dev] = v;
    *cus = v;
    return SSM_OK;
}

// ---------------------------------------------------------------------------
// Scratch memory, one growable buffer per (device, stream).  The lock is held
// for the whole enqueue so that a concurrent growth on the same stream cannot
// free a buffer that is about to be handed to a kernel.
//
// HIP graphs.  A call made while its stream is being captured records kernels
// that hold the scratch pointer for as long as the graph lives.  So:
//   * a capturing call never grows the buffer (no synchronise, no allocation):
//     if the buffer is too small it fails with SSM_ERR_CAPTURE;
//   * a buffer that was handed out during a capture is never freed when a
//     later eager call on the stream needs a larger one: it is retired and
//     kept until ssm_release_workspaces(), so replays keep valid memory.

struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
    bool captured = false;  // handed to kernels recorded into a graph
};

std::mutex g_ws_mu;
std::map<std::pair<int, uintptr_t>, Workspace> g_ws;
std::vector<std::pair<int, void *>> g_ws_retired;  // (device, buffer) a graph may still use

// Whether `s` is being captured.  An implicit capture (the legacy default
// stream while another stream captures in global mode) counts as capturing.
int stream_capturing(hipStream_t s, bool *capturing) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e == hipErrorStreamCaptureImplicit) {
        (void)hipGetLastError();
        *capturing = true;
        return SSM_OK;
    }
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    *capturing = cs != hipStreamCaptureStatusNone;
    return SSM_OK;
}

int workspace(int dev, hipStream_t s, size_t need, void **out) {
    bool capturing = false;
    int rc = stream_capturing(s, &capturing);
    if (rc) return rc;
    Workspace &w = g_ws[{dev, reinterpret_cast<uintptr_t>(s)}];
    if (w.bytes >= need) {
        if (capturing) w.captured = true;
        *out = w.ptr;
        return SSM_OK;
    }
    if (capturing)
        return fail(SSM_ERR_CAPTURE,
                    "the stream is being captured and its library scratch (%zu bytes) is smaller than this "
                    "call needs (%zu bytes); make the same call once on this stream before capturing",
                    w.bytes, need);
    if (w.ptr != nullptr) {
        if (w.captured) {
            g_ws_retired.push_back({dev, w.ptr});
        } else {
            hipError_t e = hipStreamSynchronize(s);
            if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize before growing scratch");
            e = hipFree(w.ptr);
            if (e != hipSuccess) {
                w.ptr = nullptr;
                w.bytes = 0;
                return hip_fail(e, "hipFree(scratch)");
            }
        }
        w.ptr = nullptr;
        w.bytes = 0;
        w.captured = false;
    }
    const size_t gran = (size_t)2 << 20;
    const size_t bytes = (need + gran - 1) / gran * gran;
    void *p = nullptr;
    hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        return fail(SSM_ERR_NOMEM, "hipMalloc(%zu) for scratch failed: %s", bytes, hipGetErrorString(e));
    }
    w.ptr = p;
    w.bytes = bytes;
    *out = p;
    return SSM_OK;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------

// One time step of x, delta or y (Dm * element size) must stay below 1 GiB:
// the scan kernels address a segment through 32-bit buffer offsets, and the
// planner needs at least one whole step inside a segment's 1 GiB span.
constexpr int64_t kMaxStepBytes = int64_t(1) << 30;

int check_step_bytes(int64_t Dm, int64_t es) {
    if (Dm * es >= kMaxStepBytes)
        return fail(SSM_ERR_BAD_DIM, "one time step of x (Dm = %lld values) is %lld bytes; the limit is 1 GiB",
                    (long long)Dm, (long long)(Dm * es));
    return SSM_OK;
}

constexpr unsigned kKnownFlags = SSM_DELTA_SOFTPLUS | SSM_EULER_B;

// Scratch of fixed capacity that needs no allocation (the no-allocation entry
// point): `resolve` gives its address on the current device.
struct FixedScratch {
    size_t cap;
    int (*resolve)(int dev, void **ptr);
};

// Bytes of scan scratch for S segments: converted B/C rows, segment
// summaries, entering states, and (packed sequences) restart flags.
size_t scan_scratch_bytes(int64_t S, int64_t BL, int64_t BD, int64_t N, size_t acc, bool varlen) {
    const size_t bc = align256((size_t)BL * 2 * N * acc);
    if (S <= 1) return bc;
    return bc + align256((size_t)(S - 1) * (N + 1) * BD * acc) + align256((size_t)S * N * BD * acc) +
           (varlen ? align256((size_t)S * sizeof(int)) : 0);
}

int scan_impl(const void *x, const void *delta, const float *A, const void *B, const void *C,
              const float *D, const float *h_init, void *y, float *h_final, int64_t Bsz, int64_t L,
              int64_t Dm, int64_t N, int dtype, void *stream, const int64_t *cu = nullptr,
              int64_t nseq = 0, const float *delta_bias = nullptr, unsigned flags = 0,
              const FixedScratch *fixed = nullptr) {
    const bool varlen = cu != nullptr;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32 or SSM_BF16", dtype);
    if (flags & ~kKnownFlags) return fail(SSM_ERR_BAD_OPTION, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    if (!supported_n(N)) return fail(SSM_ERR_UNSUPPORTED_N, "N = %lld; supported: 1, 2, 4, 8, 16", (long long)N);
    if (Bsz < 0 || L < 0 || Dm < 0)
        return fail(SSM_ERR_BAD_DIM, "negative size (Bsz=%lld, L=%lld, Dm=%lld)", (long long)Bsz,
                    (long long)L, (long long)Dm);
    int64_t BL, BLD, BLN, DN, BD, BDN;
    if (!mul_ok(Bsz, L, &BL) || !mul_ok(BL, Dm, &BLD) || !mul_ok(BL, N, &BLN) || !mul_ok(Dm, N, &DN) ||
        !mul_ok(Bsz, Dm, &BD) || !mul_ok(BD, N, &BDN) || BD > INT32_MAX / 2 || Bsz * ((Dm + 63) / 64) > INT32_MAX / 8)
        return fail(SSM_ERR_BAD_DIM, "sizes overflow (Bsz=%lld, L=%lld, Dm=%lld, N=%lld)", (long long)Bsz,
                    (long long)L, (long long)Dm, (long long)N);
    const int64_t es = dtype_size(dtype);
    int rc;
    if ((rc = check_step_bytes(Dm, es))) return rc;
    int64_t SDN = BDN;  // elements of h_init / h_final
    if (varlen && !mul_ok(nseq, DN, &SDN)) return fail(SSM_ERR_BAD_DIM, "nseq * Dm * N overflows");
    const Arg in[] = {{x, BLD, es, "x"}, {delta, BLD, es, "delta"}, {A, DN, 4, "A"}, {B, BLN, es, "B"},
                      {C, BLN, es, "C"}, {D, Dm, 4, "D"}, {delta_bias, delta_bias ? Dm : 0, 4, "delta_bias"},
                      {cu, varlen ? nseq + 1 : 0, 8, "cu_seqlens"}};
    const int nin = varlen ? 8 : 7;
    const Arg hi = {h_init, h_init ? SDN : 0, 4, "h_init"};
    const Arg ya = {y, BLD, es, "y"};
    const Arg hf = {h_final, h_final ? SDN : 0, 4, "h_final"};
    if ((rc = check_args(in, nin)) || (rc = check_args(&hi, 1)) || (rc = check_args(&ya, 1)) ||
        (rc = check_args(&hf, 1)))
        return rc;
    if ((rc = check_output(ya, in, nin)) || (rc = check_output(ya, &hi, 1)) || (rc = check_output(hf, in, nin)) ||
        (rc = check_output(hf, &ya, 1)))
        return rc;
    if (h_init != nullptr && h_final != nullptr && overlaps(hi, hf) &&
        (varlen || (const void *)h_init != (const void *)h_final))
        return fail(SSM_ERR_ALIAS, varlen ? "h_init overlaps h_final (not allowed for packed sequences)"
                                          : "h_init partially overlaps h_final");

    if (BD == 0 || (varlen && nseq == 0)) return ok();
    const size_t acc = ssm::scan_acc_bytes(dtype);
    if (fixed != nullptr && L > 0 && scan_scratch_bytes(1, BL, BD, N, acc, varlen) > fixed->cap)
        return fail(SSM_ERR_BAD_DIM,
                    "the call needs at least %zu bytes of scratch (Bsz * L * 2N converted B/C values); the "
                    "no-allocation entry point holds %zu",
                    scan_scratch_bytes(1, BL, BD, N, acc, varlen), fixed->cap);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // Kernel timing events are not created for the no-allocation entry point.
    auto launch = [&](int kind, auto f) -> hipError_t { return fixed ? f() : timed(kind, s, f); };

    ssm::ScanParams p;
    std::memset(&p, 0, sizeof p);
    p.x = x;
    p.delta = delta;
    p.B = B;
    p.C = C;
    p.A = A;
    p.D = D;
    p.h_init = h_init;
    p.y = y;
    p.h_final = h_final;
    p.Bsz = Bsz;
    p.L = L;
    p.Dm = Dm;
    p.waves_per_block = kWavesPerBlock;
    p.force_general = g_opt_force_general.load() ? 1 : 0;
    p.cu = cu;
    p.nseq = nseq;
    p.delta_bias = delta_bias;
    p.delta_softplus = (flags & SSM_DELTA_SOFTPLUS) ? 1 : 0;
    p.euler_b = (flags & SSM_EULER_B) ? 1 : 0;

    hipError_t e;
    if (varlen) {
        // empty sequences are never visited by the scan kernels
        e = launch(SSM_K_STATE_INIT, [&] { return ssm::launch_varlen_empty(p, (int)N, s); });
        if (e != hipSuccess) return hip_fail(e, "empty-sequence state launch");
        if (L == 0) return ok();
    }
    if (L == 0) {
        p.S = 1;
        if (h_final == nullptr) return ok();
        e = launch(SSM_K_STATE_INIT, [&] { return ssm::launch_state_init(p, (int)N, s); });
        return e == hipSuccess ? ok() : hip_fail(e, "state init launch");
    }

    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int cus = 0;
    if ((rc = device_cus(dev, &cus))) return rc;
    Plan pl = make_plan(Bsz, L, Dm, es, cus);
    if (fixed != nullptr && scan_scratch_bytes(pl.S, BL, BD, N, acc, varlen) > fixed->cap) {
        // Fewer, longer segments until the summaries fit the fixed scratch
        // (the scratch grows with S, so the first S that fits is the largest).
        int64_t S = pl.S;
        while (S > 1 && scan_scratch_bytes(S, BL, BD, N, acc, varlen) > fixed->cap) --S;
        pl.seg_len = (L + S - 1) / S;
        pl.S = (int)((L + pl.seg_len - 1) / pl.seg_len);
        if (pl.seg_len * Dm * es >= kMaxStepBytes)
            return fail(SSM_ERR_BAD_DIM,
                        "with %zu bytes of scratch the scan needs segments of %lld steps, which span 1 GiB of x "
                        "or more", fixed->cap, (long long)pl.seg_len);
    }
    p.S = pl.S;
    p.seg_len = pl.seg_len;
    p.tiles_per_b = pl.tiles_per_b;
    p.n_tiles = pl.n_tiles;

    const size_t bc_bytes = align256((size_t)BL * 2 * N * acc);
    const size_t agg_bytes = pl.S > 1 ? align256((size_t)(pl.S - 1) * (N + 1) * BD * acc) : 0;
    const size_t gin_bytes = pl.S > 1 ? align256((size_t)pl.S * N * BD * acc) : 0;
    const size_t flag_bytes = (varlen && pl.S > 1) ? align256((size_t)pl.S * sizeof(int)) : 0;

    std::unique_lock<std::mutex> lk(g_ws_mu, std::defer_lock);
    void *ws = nullptr;
    if (fixed != nullptr) {
        if ((rc = fixed->resolve(dev, &ws))) return rc;
    } else {
        lk.lock();
        if ((rc = workspace(dev, s, bc_bytes + agg_bytes + gin_bytes + flag_bytes, &ws))) return rc;
    }
    char *base = static_cast<char *>(ws);
    p.bc = base;
    p.agg = agg_bytes ? base + bc_bytes : nullptr;
    p.gin = gin_bytes ? base + bc_bytes + agg_bytes : nullptr;
    p.seg_reset = flag_bytes ? reinterpret_cast<int *>(base + bc_bytes + agg_bytes + gin_bytes) : nullptr;

    const int n = (int)N;
    if ((e = launch(SSM_K_BC_PREP, [&] { return ssm::launch_bc_prep(p, n, dtype, s); })) != hipSuccess)
        return hip_fail(e, "B/C prep launch");
    if (pl.S > 1) {
        if ((e = launch(SSM_K_SCAN_AGGREGATE, [&] { return ssm::launch_scan_aggregate(p, n, dtype, s); })) !=
            hipSuccess)
            return hip_fail(e, "segment aggregate launch");
        if ((e = launch(SSM_K_SCAN_CARRY, [&] { return ssm::launch_scan_carry(p, n, dtype, s); })) != hipSuccess)
            return hip_fail(e, "segment carry launch");
    }
    if ((e = launch(SSM_K_SCAN_OUTPUT, [&] { return ssm::launch_scan_output(p, n, dtype, s); })) != hipSuccess)
        return hip_fail(e, "segment output launch");
    return ok();
}

// Largest state of one batch row the decode step takes (2^24 fp32 values,
// 64 MiB): its kernel addresses a slice of rows through 32-bit buffer offsets.
constexpr int64_t kStepMaxRowStates = int64_t(1) << 24;

int step_impl(const void *x, const void *delta, const float *A, const void *B, const void *C,
              const float *D, float *h, void *y, int64_t Bsz, int64_t Dm, int64_t N, int dtype,
              void *stream, const float *delta_bias = nullptr, unsigned flags = 0) {
    if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32 or SSM_BF16", dtype);
    if (flags & ~kKnownFlags) return fail(SSM_ERR_BAD_OPTION, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    if (!supported_n(N)) return fail(SSM_ERR_UNSUPPORTED_N, "N = %lld; supported: 1, 2, 4, 8, 16", (long long)N);
    if (Bsz < 0 || Dm < 0)
        return fail(SSM_ERR_BAD_DIM, "negative size (Bsz=%lld, Dm=%lld)", (long long)Bsz, (long long)Dm);
    int64_t BD, BN, DN, BDN;
    if (!mul_ok(Bsz, Dm, &BD) || !mul_ok(Bsz, N, &BN) || !mul_ok(Dm, N, &DN) || !mul_ok(BD, N, &BDN) ||
        BDN > INT64_MAX / 64)
        return fail(SSM_ERR_BAD_DIM, "sizes overflow (Bsz=%lld, Dm=%lld, N=%lld)", (long long)Bsz, (long long)Dm,
                    (long long)N);
    if (DN > kStepMaxRowStates)
        return fail(SSM_ERR_BAD_DIM, "decode step: Dm*N = %lld states per batch row exceeds %lld", (long long)DN,
                    (long long)kStepMaxRowStates);
    const int64_t es = dtype_size(dtype);
    const Arg in[] = {{x, BD, es, "x"}, {delta, BD, es, "delta"}, {A, DN, 4, "A"},
                      {B, BN, es, "B"}, {C, BN, es, "C"}, {D, Dm, 4, "D"},
                      {delta_bias, delta_bias ? Dm : 0, 4, "delta_bias"}};
    const Arg ha = {h, BDN, 4, "h"};
    const Arg ya = {y, BD, es, "y"};
    int rc;
    if ((rc = check_args(in, 7)) || (rc = check_args(&ha, 1)) || (rc = check_args(&ya, 1))) return rc;
    if ((rc = check_output(ha, in, 7)) || (rc = check_output(ya, in, 7)) || (rc = check_output(ya, &ha, 1)))
        return rc;
    if (BD == 0) return ok();
    ssm::StepParams p;
    p.delta_bias = delta_bias;
    p.delta_softplus = (flags & SSM_DELTA_SOFTPLUS) ? 1 : 0;
    p.euler_b = (flags & SSM_EULER_B) ? 1 : 0;
    p.x = x;
    p.delta = delta;
    p.B = B;
    p.C = C;
    p.A = A;
    p.D = D;
    p.h = h;
    p.y = y;
    p.Bsz = Bsz;
    p.Dm = Dm;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = timed(SSM_K_STEP, s, [&] { return ssm::launch_step(p, (int)N, dtype, s); });
    return e == hipSuccess ? ok() : hip_fail(e, "decode step launch");
}

// ---------------------------------------------------------------------------
// Complex diagonal A.

int cplx_impl(const void *x, const void *delta, const float *delta_bias, const float *A, const void *B,
              const void *C, const float *D, const float *h_init, void *y, float *h_final, int64_t Bsz, int64_t L,
              int64_t Dm, int64_t N, int dtype, unsigned flags, void *stream) {
    if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32 or SSM_BF16", dtype);
    if (flags & ~kKnownFlags) return fail(SSM_ERR_BAD_OPTION, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    if (!supported_n(N)) return fail(SSM_ERR_UNSUPPORTED_N, "N = %lld; supported: 1, 2, 4, 8, 16", (long long)N);
    if (Bsz < 0 || L < 0 || Dm < 0)
        return fail(SSM_ERR_BAD_DIM, "negative size (Bsz=%lld, L=%lld, Dm=%lld)", (long long)Bsz,
                    (long long)L, (long long)Dm);
    int64_t BL, BLD, BLN, DN, BD, BDN;
    if (!mul_ok(Bsz, L, &BL) || !mul_ok(BL, Dm, &BLD) || !mul_ok(BL, N, &BLN) || !mul_ok(Dm, N, &DN) ||
        !mul_ok(Bsz, Dm, &BD) || !mul_ok(BD, N, &BDN) || BD > INT32_MAX / 2 || Bsz * ((Dm + 63) / 64) > INT32_MAX / 8 ||
        DN > INT64_MAX / 4 || BDN > INT64_MAX / 4)
        return fail(SSM_ERR_BAD_DIM, "sizes overflow (Bsz=%lld, L=%lld, Dm=%lld, N=%lld)", (long long)Bsz,
                    (long long)L, (long long)Dm, (long long)N);
    const int64_t es = dtype_size(dtype);
    int rc;
    if ((rc = check_step_bytes(Dm, es))) return rc;
    const Arg in[] = {{x, BLD, es, "x"},        {delta, BLD, es, "delta"}, {A, 2 * DN, 4, "A"},
                      {B, BLN, es, "B"},        {C, BLN, es, "C"},         {D, Dm, 4, "D"},
                      {delta_bias, delta_bias ? Dm : 0, 4, "delta_bias"}};
    const Arg hi = {h_init, h_init ? 2 * BDN : 0, 4, "h_init"};
    const Arg ya = {y, BLD, es, "y"};
    const Arg hf = {h_final, h_final ? 2 * BDN : 0, 4, "h_final"};
    if ((rc = check_args(in, 7)) || (rc = check_args(&hi, 1)) || (rc = check_args(&ya, 1)) || (rc = check_args(&hf, 1)))
        return rc;
    if ((rc = check_output(ya, in, 7)) || (rc = check_output(ya, &hi, 1)) || (rc = check_output(hf, in, 7)) ||
        (rc = check_output(hf, &ya, 1)))
        return rc;
    if (h_init != nullptr && h_final != nullptr && (const void *)h_init != (const void *)h_final && overlaps(hi, hf))
        return fail(SSM_ERR_ALIAS, "h_init partially overlaps h_final");
    if (BD == 0) return ok();
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    ssm::ScanParams p;
    std::memset(&p, 0, sizeof p);
    p.x = x;
    p.delta = delta;
    p.B = B;
    p.C = C;
    p.A = A;
    p.D = D;
    p.h_init = h_init;
    p.y = y;
    p.h_final = h_final;
    p.Bsz = Bsz;
    p.L = L;
    p.Dm = Dm;
    p.waves_per_block = kWavesPerBlock;
    p.delta_bias = delta_bias;
    p.delta_softplus = (flags & SSM_DELTA_SOFTPLUS) ? 1 : 0;
    p.euler_b = (flags & SSM_EULER_B) ? 1 : 0;
    hipError_t e;
    if (L == 0) {
        if (h_final == nullptr) return ok();
        // h_final = h_init (or zero): 2N floats per channel
        ssm::ScanParams z = p;
        z.Dm = Dm * 2;
        e = timed(SSM_K_STATE_INIT, s, [&] { return ssm::launch_state_init(z, (int)N, s); });
        return e == hipSuccess ? ok() : hip_fail(e, "state init launch");
    }
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int cus = 0;
    if ((rc = device_cus(dev, &cus))) return rc;
    const Plan pl = make_plan(Bsz, L, Dm, es, cus);
    p.S = pl.S;
    p.seg_len = pl.seg_len;
    p.tiles_per_b = pl.tiles_per_b;
    p.n_tiles = pl.n_tiles;
    const size_t acc = ssm::scan_acc_bytes(dtype);
    const size_t bc_bytes = align256((size_t)BL * 2 * N * acc);
    const size_t agg_bytes = pl.S > 1 ? align256((size_t)(pl.S - 1) * (2 * N + 1) * BD * acc) : 0;
    const size_t gin_bytes = pl.S > 1 ? align256((size_t)pl.S * 2 * N * BD * acc) : 0;
    std::lock_guard<std::mutex> lk(g_ws_mu);
    void *ws = nullptr;
    if ((rc = workspace(dev, s, bc_bytes + agg_bytes + gin_bytes, &ws))) return rc;
    char *base = static_cast<char *>(ws);
    p.bc = base;
    p.agg = agg_bytes ? base + bc_bytes : nullptr;
    p.gin = gin_bytes ? base + bc_bytes + agg_bytes : nullptr;
    const int n = (int)N;
    auto pass = [&](ssm::ScanPass ps) {
        return dtype == SSM_F32 ? ssm::cplx_pass_f32(ps, p, n, s) : ssm::cplx_pass_bf16(ps, p, n, s);
    };
    if ((e = timed(SSM_K_BC_PREP, s, [&] { return pass(ssm::ScanPass::kPrep); })) != hipSuccess)
        return hip_fail(e, "B/C conversion launch");
    if (pl.S > 1) {
        if ((e = timed(SSM_K_SCAN_AGGREGATE, s, [&] { return pass(ssm::ScanPass::kAggregate); })) != hipSuccess)
            return hip_fail(e, "segment aggregate launch");
        if ((e = timed(SSM_K_SCAN_CARRY, s, [&] { return pass(ssm::ScanPass::kCarry); })) != hipSuccess)
            return hip_fail(e, "segment carry launch");
    }
    if ((e = timed(SSM_K_SCAN_OUTPUT, s, [&] { return pass(ssm::ScanPass::kOutput); })) != hipSuccess)
        return hip_fail(e, "segment output launch");
    return ok();
}

int cplx_step_impl(const void *x, const void *delta, const float *delta_bias, const float *A, const void *B,
                   const void *C, const float *D, float *h, void *y, int64_t Bsz, int64_t Dm, int64_t N, int dtype,
                   unsigned flags, void *stream) {
    if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32 or SSM_BF16", dtype);
    if (flags & ~kKnownFlags) return fail(SSM_ERR_BAD_OPTION, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    if (!supported_n(N)) return fail(SSM_ERR_UNSUPPORTED_N, "N = %lld; supported: 1, 2, 4, 8, 16", (long long)N);
    if (Bsz < 0 || Dm < 0)
        return fail(SSM_ERR_BAD_DIM, "negative size (Bsz=%lld, Dm=%lld)", (long long)Bsz, (long long)Dm);
    int64_t BD, BN, DN, BDN;
    if (!mul_ok(Bsz, Dm, &BD) || !mul_ok(Bsz, N, &BN) || !mul_ok(Dm, N, &DN) || !mul_ok(BD, N, &BDN) ||
        BDN > INT64_MAX / 64)
        return fail(SSM_ERR_BAD_DIM, "sizes overflow (Bsz=%lld, Dm=%lld, N=%lld)", (long long)Bsz, (long long)Dm,
                    (long long)N);
    if (DN > kStepMaxRowStates / 2)
        return fail(SSM_ERR_BAD_DIM, "complex decode step: Dm*N = %lld states per batch row exceeds %lld",
                    (long long)DN, (long long)(kStepMaxRowStates / 2));
    const int64_t es = dtype_size(dtype);
    const Arg in[] = {{x, BD, es, "x"}, {delta, BD, es, "delta"}, {A, 2 * DN, 4, "A"},
                      {B, BN, es, "B"}, {C, BN, es, "C"},         {D, Dm, 4, "D"},
                      {delta_bias, delta_bias ? Dm : 0, 4, "delta_bias"}};
    const Arg ha = {h, 2 * BDN, 4, "h"};
    const Arg ya = {y, BD, es, "y"};
    int rc;
    if ((rc = check_args(in, 7)) || (rc = check_args(&ha, 1)) || (rc = check_args(&ya, 1))) return rc;
    if ((rc = check_output(ha, in, 7)) || (rc = check_output(ya, in, 7)) || (rc = check_output(ya, &ha, 1)))
        return rc;
    if (BD == 0) return ok();
    ssm::StepParams p;
    p.x = x;
    p.delta = delta;
    p.B = B;
    p.C = C;
    p.A = A;
    p.D = D;
    p.h = h;
    p.y = y;
    p.Bsz = Bsz;
    p.Dm = Dm;
    p.delta_bias = delta_bias;
    p.delta_softplus = (flags & SSM_DELTA_SOFTPLUS) ? 1 : 0;
    p.euler_b = (flags & SSM_EULER_B) ? 1 : 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = timed(SSM_K_STEP, s, [&] {
        return dtype == SSM_F32 ? ssm::cplx_step_f32(p, (int)N, s) : ssm::cplx_step_bf16(p, (int)N, s);
    });
    return e == hipSuccess ? ok() : hip_fail(e, "complex decode step launch");
}

// ---------------------------------------------------------------------------
// Backward.

// ---------------------------------------------------------------------------
// Scalar decay per head (state-space duality form).

constexpr int64_t kSsdHeadDim = 64;
constexpr int64_t kSsdChunk = 64;
constexpr int64_t kSsdHeadsPerBlock = 2;
// Blocks one CU holds at once: the output pass keeps two 4-wave blocks
// (registers), the aggregate pass about three.
constexpr int64_t kSsdOutSlotsPerCu = 2;
constexpr int64_t kSsdAggSlotsPerCu = 4;

bool ssd_supported_n(int64_t N) { return N == 32 || N == 64 || N == 128; }

// Segments of whole 64-step chunks.  A segment's chunks run one after another
// in one block, so a pass takes about (rounds of resident blocks) x (chunks
// per segment) chunk-times: the plan minimises that for the output pass plus
// the aggregate pass (which does about a third of a chunk's work, over all
// segments but the last), plus the segment states every extra segment moves
// through HBM (written by the aggregate pass, read and written by the carry,
// read by the output pass: 16 bytes per state element, counted at about
// 4 TB/s against a chunk-time of about 11 us).  SSM_OPT_SEGMENT_LEN (rounded
// up to a chunk) overrides it.
void ssd_plan(int64_t Bsz, int64_t L, int64_t H, int64_t N, int cus, int *S, int64_t *seg_len) {
    const int64_t nchunks = (L + kSsdChunk - 1) / kSsdChunk;
    const int64_t rows = Bsz * ((H + kSsdHeadsPerBlock - 1) / kSsdHeadsPerBlock);
    const int64_t c = cus > 0 ? cus : 256;
    int64_t cps = 1;
    const int64_t forced = g_opt_segment_len.load();
    if (nchunks <= 0 || rows <= 0) {
        cps = 1;
    } else if (forced > 0) {
        cps = (forced + kSsdChunk - 1) / kSsdChunk;
    } else {
        double best = -1.0;
        const int64_t smax = nchunks < 256 ? nchunks : 256;
        for (int64_t segs = 1; segs <= smax; ++segs) {
            const int64_t per = (nchunks + segs - 1) / segs;
            const int64_t sg = (nchunks + per - 1) / per;  // segments actually used
            const double out = (double)((rows * sg + kSsdOutSlotsPerCu * c - 1) / (kSsdOutSlotsPerCu * c)) * per;
            const double agg = sg > 1 ? 0.3 * (double)((rows * (sg - 1) + kSsdAggSlotsPerCu * c - 1) /
                                                        (kSsdAggSlotsPerCu * c)) * per
                                      : 0.0;
            const double states = (double)(sg - 1) * (double)(Bsz * H * kSsdHeadDim * N) / 2.75e6;
            if (best < 0 || out + agg + states < best - 1e-9) {
                best = out + agg + states;
                cps = per;
            }
        }
    }
    if (cps < 1) cps = 1;
    *seg_len = cps * kSsdChunk;
    *S = nchunks > 0 ? (int)((nchunks + cps - 1) / cps) : 1;
}

int ssd_impl(const void *x, const void *delta, const float *delta_bias, const float *A, const void *B, const void *C,
             const float *D, const float *h_init, void *y, float *h_final, int64_t Bsz, int64_t L, int64_t Dm,
             int64_t N, int64_t head_dim, int dtype, unsigned flags, void *stream) {
    if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32 or SSM_BF16", dtype);
    if (flags & ~kKnownFlags) return fail(SSM_ERR_BAD_OPTION, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    if (!ssd_supported_n(N)) return fail(SSM_ERR_UNSUPPORTED_N, "N = %lld; supported: 32, 64, 128", (long long)N);
    if (head_dim != kSsdHeadDim)
        return fail(SSM_ERR_BAD_DIM, "head_dim = %lld; supported: 64", (long long)head_dim);
    if (Bsz < 0 || L < 0 || Dm < 0)
        return fail(SSM_ERR_BAD_DIM, "negative size (Bsz=%lld, L=%lld, Dm=%lld)", (long long)Bsz,
                    (long long)L, (long long)Dm);
    if (Dm % kSsdHeadDim != 0)
        return fail(SSM_ERR_BAD_DIM, "Dm = %lld is not a multiple of head_dim = 64", (long long)Dm);
    const int64_t H = Dm / kSsdHeadDim;
    int64_t BL, BLD, BLH, BLN, BD, BDN;
    if (!mul_ok(Bsz, L, &BL) || !mul_ok(BL, Dm, &BLD) || !mul_ok(BL, H, &BLH) || !mul_ok(BL, N, &BLN) ||
        !mul_ok(Bsz, Dm, &BD) || !mul_ok(BD, N, &BDN) || Dm > ((int64_t)1 << 22) || Bsz > INT32_MAX / 2 ||
        BDN > INT64_MAX / 16)
        return fail(SSM_ERR_BAD_DIM, "sizes overflow (Bsz=%lld, L=%lld, Dm=%lld, N=%lld)", (long long)Bsz,
                    (long long)L, (long long)Dm, (long long)N);
    const int64_t es = dtype_size(dtype);
    const Arg in[] = {{x, BLD, es, "x"},        {delta, BLH, es, "delta"}, {A, H, 4, "A"},
                      {B, BLN, es, "B"},        {C, BLN, es, "C"},         {D, Dm, 4, "D"},
                      {delta_bias, delta_bias ? H : 0, 4, "delta_bias"}};
    const Arg hi = {h_init, h_init ? BDN : 0, 4, "h_init"};
    const Arg ya = {y, BLD, es, "y"};
    const Arg hf = {h_final, h_final ? BDN : 0, 4, "h_final"};
    int rc;
    if ((rc = check_args(in, 7)) || (rc = check_args(&hi, 1)) || (rc = check_args(&ya, 1)) || (rc = check_args(&hf, 1)))
        return rc;
    const Arg vec[] = {in[0], in[3], in[4], hi, ya, hf};
    for (const Arg &a : vec)
        if (a.p != nullptr && (a.lo() % 16) != 0)
            return fail(SSM_ERR_ALIGN, "%s (%p) is not 16-byte aligned", a.name, a.p);
    if ((rc = check_output(ya, in, 7)) || (rc = check_output(ya, &hi, 1)) || (rc = check_output(hf, in, 7)) ||
        (rc = check_output(hf, &ya, 1)))
        return rc;
    if (h_init != nullptr && h_final != nullptr && (const void *)h_init != (const void *)h_final && overlaps(hi, hf))
        return fail(SSM_ERR_ALIAS, "h_init partially overlaps h_final");
    if (BD == 0) return ok();
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (L == 0) {
        if (h_final == nullptr) return ok();
        ssm::ScanParams z;
        std::memset(&z, 0, sizeof z);
        z.h_init = h_init;
        z.h_final = h_final;
        z.Bsz = Bsz;
        z.Dm = Dm;
        e = timed(SSM_K_STATE_INIT, s, [&] { return ssm::launch_state_init(z, (int)N, s); });
        return e == hipSuccess ? ok() : hip_fail(e, "state init launch");
    }
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int cus = 0;
    if ((rc = device_cus(dev, &cus))) return rc;
    ssm::SsdParams p;
    std::memset(&p, 0, sizeof p);
    p.x = x;
    p.delta = delta;
    p.B = B;
    p.C = C;
    p.A = A;
    p.D = D;
    p.delta_bias = delta_bias;
    p.h_init = h_init;
    p.y = y;
    p.h_final = h_final;
    p.Bsz = Bsz;
    p.L = L;
    p.Dm = Dm;
    p.H = H;
    p.delta_softplus = (flags & SSM_DELTA_SOFTPLUS) ? 1 : 0;
    p.euler_b = (flags & SSM_EULER_B) ? 1 : 0;
    ssd_plan(Bsz, L, H, N, cus, &p.S, &p.seg_len);
    if (dtype == SSM_F32) {  // the fp64 recurrence runs over all of time at once
        p.S = 1;
        p.seg_len = L;
    }
    const int64_t blocks = Bsz * ((H + kSsdHeadsPerBlock - 1) / kSsdHeadsPerBlock) * p.S;
    if (blocks > INT32_MAX / 2)
        return fail(SSM_ERR_BAD_DIM, "too many blocks (%lld); use a longer segment", (long long)blocks);
    const size_t agg_bytes = p.S > 1 ? align256((size_t)(p.S - 1) * BDN * 4) : 0;
    const size_t dec_bytes = p.S > 1 ? align256((size_t)(p.S - 1) * Bsz * H * 4) : 0;
    const size_t gin_bytes = p.S > 1 ? align256((size_t)p.S * BDN * 4) : 0;
    std::lock_guard<std::mutex> lk(g_ws_mu);
    if (p.S > 1) {
        void *ws = nullptr;
        if ((rc = workspace(dev, s, agg_bytes + dec_bytes + gin_bytes, &ws))) return rc;
        char *base = static_cast<char *>(ws);
        p.agg = reinterpret_cast<float *>(base);
        p.dec = reinterpret_cast<float *>(base + agg_bytes);
        p.gin = reinterpret_cast<float *>(base + agg_bytes + dec_bytes);
    }
    const int n = (int)N;
    auto pass = [&](ssm::SsdPass ps) {
        return dtype == SSM_F32 ? ssm::ssd_pass_f32(ps, p, n, s) : ssm::ssd_pass_bf16(ps, p, n, s);
    };
    if (p.S > 1) {
        if ((e = timed(SSM_K_SSD_AGGREGATE, s, [&] { return pass(ssm::SsdPass::kAggregate); })) != hipSuccess)
            return hip_fail(e, "scalar-decay aggregate launch");
        if ((e = timed(SSM_K_SSD_CARRY, s, [&] { return pass(ssm::SsdPass::kCarry); })) != hipSuccess)
            return hip_fail(e, "scalar-decay carry launch");
    }
    if ((e = timed(SSM_K_SSD_OUTPUT, s, [&] { return pass(ssm::SsdPass::kOutput); })) != hipSuccess)
        return hip_fail(e, "scalar-decay output launch");
    return ok();
}

// Backward plan.  Segments have a fixed length (bwd_segment_len: 32 steps
// for bf16 storage, 16 for fp32).  A group's segments run one after another
// in one block and a CU holds two main-kernel blocks at once, so the main
// kernel takes about (rounds of resident blocks) x (segments per group): the
// plan picks the group size G that minimises it (ties: the larger G, fewer
// partial sums), with at most 256 groups.
struct BwdPlan {
    int S;
    int64_t seg_len;
    int seg_per_group;
    int groups;
    int blocks_per_row;
};

// Segments per group for `rows` blocks per group and `slots` resident blocks.
void pick_groups(BwdPlan &bp, int64_t rows, int64_t slots) {
    int64_t G = bp.S;
    int64_t best = -1;
    for (int64_t g = bp.S; g >= 1; --g) {
        const int64_t groups = (bp.S + g - 1) / g;
        if (groups > 256) break;
        const int64_t cost = (groups * rows + slots - 1) / slots * g;
        if (best < 0 || cost < best) {
            best = cost;
            G = g;
        }
    }
    bp.seg_per_group = (int)G;
    bp.groups = (int)((bp.S + G - 1) / G);
}

BwdPlan make_bwd_plan(int64_t Bsz, int64_t L, int64_t Dm, int dtype, int cus) {
    BwdPlan bp;
    bp.seg_len = ssm::bwd_segment_len(dtype);
    bp.S = L > 0 ? (int)((L + bp.seg_len - 1) / bp.seg_len) : 1;
    const int64_t tiles_per_b = (Dm + 63) / 64;
    bp.blocks_per_row = (int)((tiles_per_b + kWavesPerBlock - 1) / kWavesPerBlock);
    pick_groups(bp, Bsz * bp.blocks_per_row, 2 * (int64_t)(cus > 0 ? cus : 256));
    return bp;
}

// Complex-A backward: cbwd_segment_len() steps per segment, the main
// kernel's channel tiles per block and blocks per CU (bounded by the LDS its
// state checkpoints take) from the kernels.
BwdPlan make_cbwd_plan(int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype, int cus) {
    BwdPlan bp;
    bp.seg_len = ssm::cbwd_segment_len();
    bp.S = L > 0 ? (int)((L + bp.seg_len - 1) / bp.seg_len) : 1;
    const int64_t tiles_per_b = (Dm + 63) / 64;
    const int w = ssm::cbwd_tiles_per_block(dtype, (int)N);
    bp.blocks_per_row = (int)((tiles_per_b + w - 1) / w);
    pick_groups(bp, Bsz * bp.blocks_per_row, (int64_t)ssm::cbwd_blocks_per_cu(dtype) * (cus > 0 ? cus : 256));
    return bp;
}

int bwd_impl(const void *x, const void *delta, const float *delta_bias, const float *A, const void *B,
             const void *C, const float *D, const float *h_init, const void *dy, const float *dh_final, void *dx,
             void *ddelta, float *ddelta_bias, float *dA, float *dB, float *dC, float *dD, float *dh_init,
             int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype, unsigned flags, void *stream,
             const int64_t *cu = nullptr, int64_t nseq = 0) {
    const bool varlen = cu != nullptr;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32 or SSM_BF16", dtype);
    if (flags & ~kKnownFlags) return fail(SSM_ERR_BAD_OPTION, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    if (!supported_n(N)) return fail(SSM_ERR_UNSUPPORTED_N, "N = %lld; supported: 1, 2, 4, 8, 16", (long long)N);
    if (Bsz < 0 || L < 0 || Dm < 0)
        return fail(SSM_ERR_BAD_DIM, "negative size (Bsz=%lld, L=%lld, Dm=%lld)", (long long)Bsz,
                    (long long)L, (long long)Dm);
    int64_t BL, BLD, BLN, DN, BD, BDN;
    if (!mul_ok(Bsz, L, &BL) || !mul_ok(BL, Dm, &BLD) || !mul_ok(BL, N, &BLN) || !mul_ok(Dm, N, &DN) ||
        !mul_ok(Bsz, Dm, &BD) || !mul_ok(BD, N, &BDN) || BD > INT32_MAX / 2 || Bsz * ((Dm + 63) / 64) > INT32_MAX / 8)
        return fail(SSM_ERR_BAD_DIM, "sizes overflow (Bsz=%lld, L=%lld, Dm=%lld, N=%lld)", (long long)Bsz,
                    (long long)L, (long long)Dm, (long long)N);
    // state rows: one per batch row, or one per packed sequence
    int64_t RDN = BDN;
    if (varlen && !mul_ok(nseq, DN, &RDN)) return fail(SSM_ERR_BAD_DIM, "nseq * Dm * N overflows");
    const int64_t es = dtype_size(dtype);
    // The backward addresses a whole fixed-length segment through 32-bit
    // buffer offsets: its span must stay below 1 GiB.
    if (ssm::bwd_segment_len(dtype) * Dm * es >= kMaxStepBytes)
        return fail(SSM_ERR_BAD_DIM, "backward: a %d-step segment of x (Dm = %lld) spans %lld bytes; the limit is 1 GiB",
                    ssm::bwd_segment_len(dtype), (long long)Dm,
                    (long long)(ssm::bwd_segment_len(dtype) * Dm * es));
    const Arg in[] = {{x, BLD, es, "x"},
                      {delta, BLD, es, "delta"},
                      {A, DN, 4, "A"},
                      {B, BLN, es, "B"},
                      {C, BLN, es, "C"},
                      {D, Dm, 4, "D"},
                      {delta_bias, delta_bias ? Dm : 0, 4, "delta_bias"},
                      {h_init, h_init ? RDN : 0, 4, "h_init"},
                      {dy, BLD, es, "dy"},
                      {dh_final, dh_final ? RDN : 0, 4, "dh_final"},
                      {cu, varlen ? nseq + 1 : 0, 8, "cu_seqlens"}};
    const Arg out[] = {{dx, BLD, es, "dx"},
                       {ddelta, BLD, es, "ddelta"},
                       {ddelta_bias, ddelta_bias ? Dm : 0, 4, "ddelta_bias"},
                       {dA, DN, 4, "dA"},
                       {dB, BLN, 4, "dB"},
                       {dC, BLN, 4, "dC"},
                       {dD, Dm, 4, "dD"},
                       {dh_init, dh_init ? RDN : 0, 4, "dh_init"}};
    const int nin = varlen ? 11 : 10;
    constexpr int nout = 8;
    int rc;
    if ((rc = check_args(in, nin)) || (rc = check_args(out, nout))) return rc;
    for (int i = 0; i < nout; ++i) {
        if ((rc = check_output(out[i], in, nin))) return rc;
        for (int j = 0; j < i; ++j)
            if (overlaps(out[i], out[j])) return fail(SSM_ERR_ALIAS, "%s overlaps %s", out[i].name, out[j].name);
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (BD == 0 || L == 0) {
        // nothing flows: parameter gradients are zero, dh_init = dh_final
        e = timed(SSM_K_STATE_INIT, s, [&] {
            hipError_t r = ssm::launch_fill(dA, DN, 0.f, s);
            if (r == hipSuccess) r = ssm::launch_fill(dD, Dm, 0.f, s);
            if (r == hipSuccess) r = ssm::launch_fill(ddelta_bias, ddelta_bias ? Dm : 0, 0.f, s);
            // dB, dC are sums over channels: zero when there are none
            if (r == hipSuccess) r = ssm::launch_fill(dB, BLN, 0.f, s);
            if (r == hipSuccess) r = ssm::launch_fill(dC, BLN, 0.f, s);
            if (r == hipSuccess && dh_init != nullptr) {
                // (packed: every sequence is empty, or Dm is 0)
                ssm::ScanParams z;
                std::memset(&z, 0, sizeof z);
                z.Bsz = varlen ? nseq : Bsz;
                z.Dm = Dm;
                z.h_init = dh_final;
                z.h_final = dh_init;
                r = ssm::launch_state_init(z, (int)N, s);
            }
            return r;
        });
        return e == hipSuccess ? ok() : hip_fail(e, "zero-size backward");
    }

    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int cus = 0;
    if ((rc = device_cus(dev, &cus))) return rc;

    ssm::BwdParams q;
    std::memset(&q, 0, sizeof q);
    ssm::ScanParams &p = q.f;
    p.x = x;
    p.delta = delta;
    p.B = B;
    p.C = C;
    p.A = A;
    p.D = D;
    p.h_init = h_init;
    p.Bsz = Bsz;
    p.L = L;
    p.Dm = Dm;
    p.waves_per_block = kWavesPerBlock;
    p.force_general = g_opt_force_general.load() ? 1 : 0;
    p.cu = cu;
    p.nseq = nseq;
    p.delta_bias = delta_bias;
    p.delta_softplus = (flags & SSM_DELTA_SOFTPLUS) ? 1 : 0;
    p.euler_b = (flags & SSM_EULER_B) ? 1 : 0;
    p.seg_len = ssm::bwd_segment_len(dtype);
    p.S = (int)((L + p.seg_len - 1) / p.seg_len);
    p.tiles_per_b = (int)((Dm + 63) / 64);
    p.n_tiles = (int)(Bsz * p.tiles_per_b);
    q.dy = dy;
    q.dh_final = dh_final;
    q.dx = dx;
    q.ddelta = ddelta;
    q.ddelta_bias = ddelta_bias;
    q.dA = dA;
    q.dB = dB;
    q.dC = dC;
    q.dD = dD;
    q.dh_init = dh_init;
    const BwdPlan bp = make_bwd_plan(Bsz, L, Dm, dtype, cus);
    q.blocks_per_row = bp.blocks_per_row;
    q.seg_per_group = bp.seg_per_group;
    q.n_groups = bp.groups;
    if ((int64_t)q.n_groups * Bsz * q.blocks_per_row >= ((int64_t)1 << 31) ||
        (int64_t)((p.n_tiles + kWavesPerBlock - 1) / kWavesPerBlock) * p.S >= ((int64_t)1 << 31))
        return fail(SSM_ERR_BAD_DIM, "backward grid too large (Bsz=%lld, L=%lld, Dm=%lld)", (long long)Bsz,
                    (long long)L, (long long)Dm);

    const size_t acc = ssm::scan_acc_bytes(dtype);
    const size_t S = (size_t)p.S;
    const size_t sz_bc = align256((size_t)BL * 2 * N * acc);
    const size_t sz_agg = align256((S > 1 ? S - 1 : 0) * (N + 1) * BD * acc);
    const size_t sz_gin = align256(S * N * BD * acc);
    const size_t sz_ragg = align256(S * (N + 1) * BD * acc);
    const size_t sz_gout = align256((size_t)q.n_groups * N * BD * acc);
    const size_t sz_pbc = align256((size_t)2 * q.blocks_per_row * 2 * BLN * acc);
    const size_t sz_pa = align256((size_t)q.n_groups * BD * N * acc);
    const size_t sz_pd = align256((size_t)q.n_groups * BD * 2 * acc);
    const size_t sz_pon = align256((size_t)2 * q.blocks_per_row * Bsz * q.n_groups * sizeof(int));
    const size_t sz_res = varlen ? align256(S * sizeof(int)) : 0;  // forward reset flags; start masks

    std::lock_guard<std::mutex> lk(g_ws_mu);
    void *ws = nullptr;
    if ((rc = workspace(dev, s,
                        sz_bc + sz_agg + sz_gin + sz_ragg + sz_gout + sz_pbc + sz_pa + sz_pd + sz_pon + 2 * sz_res,
                        &ws)))
        return rc;
    char *base = static_cast<char *>(ws);
    p.bc = base;
    base += sz_bc;
    p.agg = sz_agg ? base : nullptr;
    base += sz_agg;
    p.gin = base;
    base += sz_gin;
    q.ragg = base;
    base += sz_ragg;
    q.gout = base;
    base += sz_gout;
    q.part_bc = base;
    base += sz_pbc;
    q.part_a = base;
    base += sz_pa;
    q.part_d = base;
    base += sz_pd;
    q.part_on = reinterpret_cast<int *>(base);
    base += sz_pon;
    p.seg_reset = varlen ? reinterpret_cast<int *>(base) : nullptr;
    base += sz_res;
    q.seg_starts = varlen ? reinterpret_cast<uint32_t *>(base) : nullptr;

    const int n = (int)N;
    auto bwd = [&](ssm::BwdPass pass) {
        if (dtype == SSM_F32)
            return varlen ? ssm::bwd_pass_f32_packed(pass, q, n, s) : ssm::bwd_pass_f32(pass, q, n, s);
        return varlen ? ssm::bwd_pass_bf16_packed(pass, q, n, s) : ssm::bwd_pass_bf16(pass, q, n, s);
    };
    if ((e = timed(SSM_K_BC_PREP, s, [&] { return ssm::launch_bc_prep(p, n, dtype, s); })) != hipSuccess)
        return hip_fail(e, "B/C conversion launch");
    if (varlen && (e = timed(SSM_K_STATE_INIT, s, [&] { return bwd(ssm::BwdPass::kStarts); })) != hipSuccess)
        return hip_fail(e, "sequence-start launch");
    if (p.S > 1) {
        if ((e = timed(SSM_K_SCAN_AGGREGATE, s, [&] { return ssm::launch_scan_aggregate(p, n, dtype, s); })) !=
            hipSuccess)
            return hip_fail(e, "forward aggregate launch");
        if ((e = timed(SSM_K_SCAN_CARRY, s, [&] { return ssm::launch_scan_carry(p, n, dtype, s); })) != hipSuccess)
            return hip_fail(e, "forward carry launch");
        if ((e = timed(SSM_K_BWD_AGGREGATE, s, [&] { return bwd(ssm::BwdPass::kAggregate); })) != hipSuccess)
            return hip_fail(e, "backward aggregate launch");
    }
    if ((e = timed(SSM_K_BWD_CARRY, s, [&] { return bwd(ssm::BwdPass::kCarry); })) != hipSuccess)
        return hip_fail(e, "backward carry launch");
    if ((e = timed(SSM_K_BWD_MAIN, s, [&] { return bwd(ssm::BwdPass::kMain); })) != hipSuccess)
        return hip_fail(e, "backward main launch");
    if ((e = timed(SSM_K_BWD_REDUCE, s, [&] { return bwd(ssm::BwdPass::kReduce); })) != hipSuccess)
        return hip_fail(e, "backward reduction launch");
    if (varlen && dh_init != nullptr) {
        // empty sequences: dh_init = dh_final (their final state is their initial one)
        ssm::ScanParams z;
        std::memset(&z, 0, sizeof z);
        z.Dm = Dm;
        z.cu = cu;
        z.nseq = nseq;
        z.h_init = dh_final;
        z.h_final = dh_init;
        if ((e = timed(SSM_K_STATE_INIT, s, [&] { return ssm::launch_varlen_empty(z, n, s); })) != hipSuccess)
            return hip_fail(e, "empty-sequence launch");
    }
    return ok();
}

// Complex diagonal A: A, dA [Dm][N][2]; h_init, dh_final, dh_init
// [Bsz][Dm][N][2] (re, im pairs).  The forward's aggregate and carry passes
// (cplx_pass) give the state entering every backward segment.
int cbwd_impl(const void *x, const void *delta, const float *delta_bias, const float *A, const void *B,
              const void *C, const float *D, const float *h_init, const void *dy, const float *dh_final, void *dx,
              void *ddelta, float *ddelta_bias, float *dA, float *dB, float *dC, float *dD, float *dh_init,
              int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype, unsigned flags, void *stream) {
    if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d is not SSM_F32 or SSM_BF16", dtype);
    if (flags & ~kKnownFlags) return fail(SSM_ERR_BAD_OPTION, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    if (!supported_n(N)) return fail(SSM_ERR_UNSUPPORTED_N, "N = %lld; supported: 1, 2, 4, 8, 16", (long long)N);
    if (Bsz < 0 || L < 0 || Dm < 0)
        return fail(SSM_ERR_BAD_DIM, "negative size (Bsz=%lld, L=%lld, Dm=%lld)", (long long)Bsz,
                    (long long)L, (long long)Dm);
    int64_t BL, BLD, BLN, DN, BD, BDN;
    if (!mul_ok(Bsz, L, &BL) || !mul_ok(BL, Dm, &BLD) || !mul_ok(BL, N, &BLN) || !mul_ok(Dm, N, &DN) ||
        !mul_ok(Bsz, Dm, &BD) || !mul_ok(BD, N, &BDN) || BD > INT32_MAX / 2 || Bsz * ((Dm + 63) / 64) > INT32_MAX / 8 ||
        DN > INT64_MAX / 4 || BDN > INT64_MAX / 4)
        return fail(SSM_ERR_BAD_DIM, "sizes overflow (Bsz=%lld, L=%lld, Dm=%lld, N=%lld)", (long long)Bsz,
                    (long long)L, (long long)Dm, (long long)N);
    const int64_t es = dtype_size(dtype);
    const int seg = ssm::cbwd_segment_len();
    if (seg * Dm * es >= kMaxStepBytes)
        return fail(SSM_ERR_BAD_DIM, "backward: a %d-step segment of x (Dm = %lld) spans %lld bytes; the limit is 1 GiB",
                    seg, (long long)Dm, (long long)(seg * Dm * es));
    const Arg in[] = {{x, BLD, es, "x"},
                      {delta, BLD, es, "delta"},
                      {A, 2 * DN, 4, "A"},
                      {B, BLN, es, "B"},
                      {C, BLN, es, "C"},
                      {D, Dm, 4, "D"},
                      {delta_bias, delta_bias ? Dm : 0, 4, "delta_bias"},
                      {h_init, h_init ? 2 * BDN : 0, 4, "h_init"},
                      {dy, BLD, es, "dy"},
                      {dh_final, dh_final ? 2 * BDN : 0, 4, "dh_final"}};
    const Arg out[] = {{dx, BLD, es, "dx"},
                       {ddelta, BLD, es, "ddelta"},
                       {ddelta_bias, ddelta_bias ? Dm : 0, 4, "ddelta_bias"},
                       {dA, 2 * DN, 4, "dA"},
                       {dB, BLN, 4, "dB"},
                       {dC, BLN, 4, "dC"},
                       {dD, Dm, 4, "dD"},
                       {dh_init, dh_init ? 2 * BDN : 0, 4, "dh_init"}};
    constexpr int nin = 10, nout = 8;
    int rc;
    if ((rc = check_args(in, nin)) || (rc = check_args(out, nout))) return rc;
    for (int i = 0; i < nout; ++i) {
        if ((rc = check_output(out[i], in, nin))) return rc;
        for (int j = 0; j < i; ++j)
            if (overlaps(out[i], out[j])) return fail(SSM_ERR_ALIAS, "%s overlaps %s", out[i].name, out[j].name);
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (BD == 0 || L == 0) {
        e = timed(SSM_K_STATE_INIT, s, [&] {
            hipError_t r = ssm::launch_fill(dA, 2 * DN, 0.f, s);
            if (r == hipSuccess) r = ssm::launch_fill(dD, Dm, 0.f, s);
            if (r == hipSuccess) r = ssm::launch_fill(ddelta_bias, ddelta_bias ? Dm : 0, 0.f, s);
            if (r == hipSuccess) r = ssm::launch_fill(dB, BLN, 0.f, s);
            if (r == hipSuccess) r = ssm::launch_fill(dC, BLN, 0.f, s);
            if (r == hipSuccess && dh_init != nullptr) {
                // dh_init = dh_final (or zero), 2N floats per channel
                ssm::ScanParams z;
                std::memset(&z, 0, sizeof z);
                z.Bsz = Bsz;
                z.Dm = Dm * 2;
                z.h_init = dh_final;
                z.h_final = dh_init;
                r = ssm::launch_state_init(z, (int)N, s);
            }
            return r;
        });
        return e == hipSuccess ? ok() : hip_fail(e, "zero-size backward");
    }

    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int cus = 0;
    if ((rc = device_cus(dev, &cus))) return rc;

    ssm::BwdParams q;
    std::memset(&q, 0, sizeof q);
    ssm::ScanParams &p = q.f;
    p.x = x;
    p.delta = delta;
    p.B = B;
    p.C = C;
    p.A = A;
    p.D = D;
    p.h_init = h_init;
    p.Bsz = Bsz;
    p.L = L;
    p.Dm = Dm;
    p.waves_per_block = kWavesPerBlock;
    p.delta_bias = delta_bias;
    p.delta_softplus = (flags & SSM_DELTA_SOFTPLUS) ? 1 : 0;
    p.euler_b = (flags & SSM_EULER_B) ? 1 : 0;
    const BwdPlan bp = make_cbwd_plan(Bsz, L, Dm, N, dtype, cus);
    p.seg_len = bp.seg_len;
    p.S = bp.S;
    p.tiles_per_b = (int)((Dm + 63) / 64);
    p.n_tiles = (int)(Bsz * p.tiles_per_b);
    q.dy = dy;
    q.dh_final = dh_final;
    q.dx = dx;
    q.ddelta = ddelta;
    q.ddelta_bias = ddelta_bias;
    q.dA = dA;
    q.dB = dB;
    q.dC = dC;
    q.dD = dD;
    q.dh_init = dh_init;
    q.blocks_per_row = bp.blocks_per_row;
    q.seg_per_group = bp.seg_per_group;
    q.n_groups = bp.groups;
    if ((int64_t)q.n_groups * Bsz * q.blocks_per_row >= ((int64_t)1 << 31) ||
        (int64_t)((p.n_tiles + kWavesPerBlock - 1) / kWavesPerBlock) * p.S >= ((int64_t)1 << 31))
        return fail(SSM_ERR_BAD_DIM, "backward grid too large (Bsz=%lld, L=%lld, Dm=%lld)", (long long)Bsz,
                    (long long)L, (long long)Dm);

    const size_t acc = ssm::scan_acc_bytes(dtype);
    const size_t S = (size_t)p.S;
    const size_t sz_bc = align256((size_t)BL * 2 * N * acc);
    const size_t sz_agg = align256((S > 1 ? S - 1 : 0) * (2 * N + 1) * BD * acc);
    const size_t sz_gin = align256(S * 2 * N * BD * acc);
    const size_t sz_ragg = align256(S * (2 * N + 1) * BD * acc);
    const size_t sz_gout = align256((size_t)q.n_groups * 2 * N * BD * acc);
    const size_t sz_pbc = align256((size_t)q.blocks_per_row * 2 * BLN * acc);
    const size_t sz_pa = align256((size_t)q.n_groups * BD * 2 * N * acc);
    const size_t sz_pd = align256((size_t)q.n_groups * BD * 2 * acc);

    std::lock_guard<std::mutex> lk(g_ws_mu);
    void *ws = nullptr;
    if ((rc = workspace(dev, s, sz_bc + sz_agg + sz_gin + sz_ragg + sz_gout + sz_pbc + sz_pa + sz_pd, &ws)))
        return rc;
    char *base = static_cast<char *>(ws);
    p.bc = base;
    base += sz_bc;
    p.agg = sz_agg ? base : nullptr;
    base += sz_agg;
    p.gin = base;
    base += sz_gin;
    q.ragg = base;
    base += sz_ragg;
    q.gout = base;
    base += sz_gout;
    q.part_bc = base;
    base += sz_pbc;
    q.part_a = base;
    base += sz_pa;
    q.part_d = base;

    const int n = (int)N;
    auto fwd = [&](ssm::ScanPass ps) {
        return dtype == SSM_F32 ? ssm::cplx_pass_f32(ps, p, n, s) : ssm::cplx_pass_bf16(ps, p, n, s);
    };
    auto bwd = [&](ssm::BwdPass pass) {
        return dtype == SSM_F32 ? ssm::cbwd_pass_f32(pass, q, n, s) : ssm::cbwd_pass_bf16(pass, q, n, s);
    };
    if ((e = timed(SSM_K_BC_PREP, s, [&] { return fwd(ssm::ScanPass::kPrep); })) != hipSuccess)
        return hip_fail(e, "B/C conversion launch");
    if (p.S > 1) {
        // one pass gives the segment summaries of both directions
        if ((e = timed(SSM_K_BWD_AGGREGATE, s, [&] { return bwd(ssm::BwdPass::kAggregate); })) != hipSuccess)
            return hip_fail(e, "segment summary launch");
        if ((e = timed(SSM_K_SCAN_CARRY, s, [&] { return fwd(ssm::ScanPass::kCarry); })) != hipSuccess)
            return hip_fail(e, "forward carry launch");
    }
    if ((e = timed(SSM_K_BWD_CARRY, s, [&] { return bwd(ssm::BwdPass::kCarry); })) != hipSuccess)
        return hip_fail(e, "backward carry launch");
    if ((e = timed(SSM_K_BWD_MAIN, s, [&] { return bwd(ssm::BwdPass::kMain); })) != hipSuccess)
        return hip_fail(e, "backward main launch");
    if ((e = timed(SSM_K_BWD_REDUCE, s, [&] { return bwd(ssm::BwdPass::kReduce); })) != hipSuccess)
        return hip_fail(e, "backward reduction launch");
    return ok();
}

}  // namespace

namespace ssm {

int scan_fwd_fixed_scratch(const void *x, const void *delta, const float *A, const void *B, const void *C,
                           const float *D, const float *h_init, void *y, float *h_final, int64_t Bsz, int64_t L,
                           int64_t Dm, int64_t N, int dtype, void *stream, size_t cap,
                           int (*resolve)(int dev, void **ptr)) {
    const FixedScratch fs = {cap, resolve};
    return scan_impl(x, delta, A, B, C, D, h_init, y, h_final, Bsz, L, Dm, N, dtype, stream, nullptr, 0, nullptr,
                     0, &fs);
}

int set_error(int code, const char *msg) { return fail(code, "%s", msg); }

}  // namespace ssm

extern "C" {

int ssm_scan_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, void *y, float *h_final, int64_t Bsz, int64_t L, int64_t Dm, int64_t N,
                 int dtype, void *stream) {
    return scan_impl(x, delta, A, B, C, D, nullptr, y, h_final, Bsz, L, Dm, N, dtype, stream);
}

int ssm_scan_fwd_ex(const void *x, const void *delta, const float *A, const void *B, const void *C,
                    const float *D, const float *h_init, void *y, float *h_final, int64_t Bsz, int64_t L,
                    int64_t Dm, int64_t N, int dtype, void *stream) {
    return scan_impl(x, delta, A, B, C, D, h_init, y, h_final, Bsz, L, Dm, N, dtype, stream);
}

int ssm_scan_varlen_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C,
                        const float *D, const int64_t *cu_seqlens, int64_t nseq, const float *h_init,
                        void *y, float *h_final, int64_t L, int64_t Dm, int64_t N, int dtype, void *stream) {
    if (nseq < 0) return fail(SSM_ERR_BAD_DIM, "nseq = %lld < 0", (long long)nseq);
    if (nseq == 0 && L > 0) return fail(SSM_ERR_BAD_DIM, "nseq = 0 but L = %lld", (long long)L);
    if (cu_seqlens == nullptr) return fail(SSM_ERR_NULLPTR, "cu_seqlens is NULL");
    return scan_impl(x, delta, A, B, C, D, h_init, y, h_final, 1, L, Dm, N, dtype, stream, cu_seqlens, nseq);
}

int ssm_scan_fused_fwd(const void *x, const void *delta, const float *delta_bias, const float *A,
                       const void *B, const void *C, const float *D, const int64_t *cu_seqlens, int64_t nseq,
                       const float *h_init, void *y, float *h_final, int64_t Bsz, int64_t L, int64_t Dm,
                       int64_t N, int dtype, unsigned flags, void *stream) {
    if (cu_seqlens != nullptr) {
        if (Bsz != 1) return fail(SSM_ERR_BAD_DIM, "packed sequences need Bsz = 1 (got %lld)", (long long)Bsz);
        if (nseq < 0) return fail(SSM_ERR_BAD_DIM, "nseq = %lld < 0", (long long)nseq);
        if (nseq == 0 && L > 0) return fail(SSM_ERR_BAD_DIM, "nseq = 0 but L = %lld", (long long)L);
    }
    return scan_impl(x, delta, A, B, C, D, h_init, y, h_final, Bsz, L, Dm, N, dtype, stream, cu_seqlens,
                     cu_seqlens ? nseq : 0, delta_bias, flags);
}

int ssm_step_fused(const void *x, const void *delta, const float *delta_bias, const float *A, const void *B,
                   const void *C, const float *D, float *h, void *y, int64_t Bsz, int64_t Dm, int64_t N, int dtype,
                   unsigned flags, void *stream) {
    return step_impl(x, delta, A, B, C, D, h, y, Bsz, Dm, N, dtype, stream, delta_bias, flags);
}

int ssm_scan_bwd(const void *x, const void *delta, const float *delta_bias, const float *A, const void *B,
                 const void *C, const float *D, const float *h_init, const void *dy, const float *dh_final,
                 void *dx, void *ddelta, float *ddelta_bias, float *dA, float *dB, float *dC, float *dD,
                 float *dh_init, int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype, unsigned flags,
                 void *stream) {
    return bwd_impl(x, delta, delta_bias, A, B, C, D, h_init, dy, dh_final, dx, ddelta, ddelta_bias, dA, dB, dC,
                    dD, dh_init, Bsz, L, Dm, N, dtype, flags, stream);
}

int ssm_scan_varlen_bwd(const void *x, const void *delta, const float *delta_bias, const float *A, const void *B,
                        const void *C, const float *D, const int64_t *cu_seqlens, int64_t nseq, const float *h_init,
                        const void *dy, const float *dh_final, void *dx, void *ddelta, float *ddelta_bias,
                        float *dA, float *dB, float *dC, float *dD, float *dh_init, int64_t L, int64_t Dm,
                        int64_t N, int dtype, unsigned flags, void *stream) {
    if (nseq < 0) return fail(SSM_ERR_BAD_DIM, "nseq = %lld < 0", (long long)nseq);
    if (nseq == 0 && L > 0) return fail(SSM_ERR_BAD_DIM, "nseq = 0 but L = %lld", (long long)L);
    if (cu_seqlens == nullptr) return fail(SSM_ERR_NULLPTR, "cu_seqlens is NULL");
    return bwd_impl(x, delta, delta_bias, A, B, C, D, h_init, dy, dh_final, dx, ddelta, ddelta_bias, dA, dB, dC,
                    dD, dh_init, 1, L, Dm, N, dtype, flags, stream, cu_seqlens, nseq);
}

int ssm_scan_complex_fwd(const void *x, const void *delta, const float *delta_bias, const float *A, const void *B,
                         const void *C, const float *D, const float *h_init, void *y, float *h_final, int64_t Bsz,
                         int64_t L, int64_t Dm, int64_t N, int dtype, unsigned flags, void *stream) {
    return cplx_impl(x, delta, delta_bias, A, B, C, D, h_init, y, h_final, Bsz, L, Dm, N, dtype, flags, stream);
}

int ssm_scan_complex_bwd(const void *x, const void *delta, const float *delta_bias, const float *A, const void *B,
                         const void *C, const float *D, const float *h_init, const void *dy, const float *dh_final,
                         void *dx, void *ddelta, float *ddelta_bias, float *dA, float *dB, float *dC, float *dD,
                         float *dh_init, int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype, unsigned flags,
                         void *stream) {
    return cbwd_impl(x, delta, delta_bias, A, B, C, D, h_init, dy, dh_final, dx, ddelta, ddelta_bias, dA, dB, dC, dD,
                     dh_init, Bsz, L, Dm, N, dtype, flags, stream);
}

int ssm_scan_ssd_fwd(const void *x, const void *delta, const float *delta_bias, const float *A, const void *B,
                     const void *C, const float *D, const float *h_init, void *y, float *h_final, int64_t Bsz,
                     int64_t L, int64_t Dm, int64_t N, int64_t head_dim, int dtype, unsigned flags, void *stream) {
    return ssd_impl(x, delta, delta_bias, A, B, C, D, h_init, y, h_final, Bsz, L, Dm, N, head_dim, dtype, flags,
                    stream);
}

int ssm_step_complex(const void *x, const void *delta, const float *delta_bias, const float *A, const void *B,
                     const void *C, const float *D, float *h, void *y, int64_t Bsz, int64_t Dm, int64_t N, int dtype,
                     unsigned flags, void *stream) {
    return cplx_step_impl(x, delta, delta_bias, A, B, C, D, h, y, Bsz, Dm, N, dtype, flags, stream);
}

int ssm_step(const void *x, const void *delta, const float *A, const void *B, const void *C,
             const float *D, float *h, void *y, int64_t Bsz, int64_t Dm, int64_t N, void *stream) {
    return step_impl(x, delta, A, B, C, D, h, y, Bsz, Dm, N, SSM_BF16, stream);
}

int ssm_step_ex(const void *x, const void *delta, const float *A, const void *B, const void *C,
                const float *D, float *h, void *y, int64_t Bsz, int64_t Dm, int64_t N, int dtype,
                void *stream) {
    return step_impl(x, delta, A, B, C, D, h, y, Bsz, Dm, N, dtype, stream);
}

const char *ssm_strerror(int code) {
    switch (code) {
        case SSM_OK: return "success";
        case SSM_ERR_NULLPTR: return "a non-empty tensor has a NULL pointer";
        case SSM_ERR_BAD_DIM: return "invalid or overflowing size";
        case SSM_ERR_BAD_DTYPE: return "unsupported dtype";
        case SSM_ERR_UNSUPPORTED_N: return "unsupported state size N";
        case SSM_ERR_ALIGN: return "pointer not aligned to its element size";
        case SSM_ERR_ALIAS: return "an output overlaps another argument";
        case SSM_ERR_NOMEM: return "scratch allocation failed";
        case SSM_ERR_HIP: return "HIP runtime error";
        case SSM_ERR_BAD_OPTION: return "unknown option or invalid option value";
        case SSM_ERR_CAPTURE: return "scratch too small for a call on a capturing stream";
        default: return "unknown status code";
    }
}

const char *ssm_last_error(void) { return g_last_error.c_str(); }

int ssm_version(void) { return kVersion; }

int ssm_set_option(int option, int64_t value) {
    switch (option) {
        case SSM_OPT_SEGMENT_LEN:
            if (value < 0) return fail(SSM_ERR_BAD_OPTION, "segment length %lld < 0", (long long)value);
            g_opt_segment_len.store(value);
            return ok();
        case SSM_OPT_FORCE_GENERAL:
            if (value != 0 && value != 1) return fail(SSM_ERR_BAD_OPTION, "force-general must be 0 or 1");
            g_opt_force_general.store(value);
            return ok();
        case SSM_OPT_PROFILE:
            if (value != 0 && value != 1) return fail(SSM_ERR_BAD_OPTION, "profile must be 0 or 1");
            g_opt_profile.store(value);
            return ok();
        case SSM_OPT_STEP_CHANNELS:
            if (value != 1 && value != 2 && value != 4)
                return fail(SSM_ERR_BAD_OPTION, "step channels per thread must be 1, 2 or 4");
            g_opt_step_channels.store(value);
            ssm::set_step_unroll((int)value);
            return ok();
        default:
            return fail(SSM_ERR_BAD_OPTION, "unknown option %d", option);
    }
}

int64_t ssm_get_option(int option) {
    switch (option) {
        case SSM_OPT_SEGMENT_LEN: return g_opt_segment_len.load();
        case SSM_OPT_FORCE_GENERAL: return g_opt_force_general.load();
        case SSM_OPT_PROFILE: return g_opt_profile.load();
        case SSM_OPT_STEP_CHANNELS: return g_opt_step_channels.load();
        default: return -1;
    }
}

int ssm_scan_plan(int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype, int compute_units,
                  int64_t *segments, int64_t *segment_len) {
    if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d", dtype);
    if (!supported_n(N)) return fail(SSM_ERR_UNSUPPORTED_N, "N = %lld", (long long)N);
    if (Bsz < 0 || L < 0 || Dm < 0) return fail(SSM_ERR_BAD_DIM, "negative size");
    if (segments == nullptr || segment_len == nullptr) return fail(SSM_ERR_NULLPTR, "output pointer is NULL");
    int cus = compute_units;
    if (cus <= 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        int rc = device_cus(dev, &cus);
        if (rc) return rc;
    }
    const Plan pl = make_plan(Bsz, L, Dm, dtype_size(dtype), cus);
    *segments = pl.S;
    *segment_len = pl.seg_len;
    return ok();
}

int ssm_scan_bwd_plan(int64_t Bsz, int64_t L, int64_t Dm, int64_t N, int dtype, int compute_units,
                      int64_t *segments, int64_t *segment_len, int64_t *seg_per_group, int64_t *groups) {
    if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_ERR_BAD_DTYPE, "dtype %d", dtype);
    if (!supported_n(N)) return fail(SSM_ERR_UNSUPPORTED_N, "N = %lld", (long long)N);
    if (Bsz < 0 || L < 0 || Dm < 0) return fail(SSM_ERR_BAD_DIM, "negative size");
    if (segments == nullptr || segment_len == nullptr || seg_per_group == nullptr || groups == nullptr)
        return fail(SSM_ERR_NULLPTR, "output pointer is NULL");
    int cus = compute_units;
    if (cus <= 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        int rc = device_cus(dev, &cus);
        if (rc) return rc;
    }
    const BwdPlan bp = make_bwd_plan(Bsz, L, Dm, dtype, cus);
    *segments = bp.S;
    *segment_len = bp.seg_len;
    *seg_per_group = bp.seg_per_group;
    *groups = bp.groups;
    return ok();
}

int ssm_profile_read(double *total_ms, int64_t *launches, int n) {
    std::vector<ProfRec> recs;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        recs.swap(g_prof);
    }
    for (int k = 0; k < n; ++k) {
        if (total_ms) total_ms[k] = 0.0;
        if (launches) launches[k] = 0;
    }
    int rc = SSM_OK;
    for (const ProfRec &r : recs) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess && rc == SSM_OK) rc = hip_fail(e, "reading kernel timing events");
        if (e == hipSuccess && r.kind >= 0 && r.kind < n) {
            if (total_ms) total_ms[r.kind] += ms;
            if (launches) launches[r.kind] += 1;
        }
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    return rc == SSM_OK ? ok() : rc;
}

int ssm_release_workspaces(void) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    int rc = SSM_OK;
    auto release = [&](int dev, void *ptr) {
        int cur = 0;
        if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(dev) == hipSuccess) {
            hipError_t e = hipFree(ptr);
            if (e != hipSuccess && rc == SSM_OK) rc = hip_fail(e, "hipFree(scratch)");
            (void)hipSetDevice(cur);
        }
    };
    for (auto &kv : g_ws)
        if (kv.second.ptr != nullptr) release(kv.first.first, kv.second.ptr);
    for (auto &r : g_ws_retired) release(r.first, r.second);
    g_ws.clear();
    g_ws_retired.clear();
    return rc == SSM_OK ? ok() : rc;
}

}  // extern "C"
