// C ABI of tilegemm: argument validation, kernel-configuration choice and launch.
//
// The call shape follows the pages' problem statement (the mhpq.cn page,
// section 3.2: the caller allocates A, B and C and launches kernel(A, B, C);
// section 3.4 checks the inner dimensions first) and the blog.hotdry.top page's
// per-shape kernels (matmul(M, N, K, ...)).  Shapes arrive at run time here;
// tile sizes, wave layout, stage count and swizzle group are compile-time
// constants of each compiled configuration, chosen per call from a table that
// the offline sweep (tiled_dense_gemm_07_amd/sweep.py) writes.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/tilegemm.h"
#include "tg_configs.h"
#include "tg_kernel.h"

// Scratch of tg_gemm_splitk_noalloc: the split-K arrival counters and fp32
// partial tiles, in a fixed device array instead of caller memory.  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code `scratch` is only the host-side handle of the symbol: its device
// address comes from hipGetSymbolAddress (per device, in scratch_of_device).
static __device__ __attribute__((aligned(256))) char scratch[TG_SPLITK_SCRATCH_BYTES];

// Zero n int32 counters (a fill kernel, so that a captured graph holds no
// memset node).
__global__ void tg_clear_counters(int* counters, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        counters[i] = 0;
}

namespace {

// Device address of `scratch` on the calling thread's current device,
// looked up once per device.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

tg_status scratch_of_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TG_ERR_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return TG_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return TG_OK;
}

using tg::Config;
using tg::ConfigList;

// One row of the selection table the offline sweep writes (tg_tuned.inc).
// exact != 0: the best configuration measured for exactly this shape.
// exact == 0: one of the best configurations measured at the representative
// shape (M, N, K) of a shape bucket, with its measured time; a call whose
// nearest representative this is picks among them by the cost model below.
struct TunedEntry {
    int op;
    int dtype;
    int64_t M, N, K;
    const char* config;  // configuration name, as config_name() prints it
    int group_m;         // swizzle group to launch with (0: the configuration's default)
    double ms;           // measured time at (M, N, K)
    int per_cu;          // workgroups of this configuration one compute unit holds
    int exact;
};

#include "tg_tuned.inc"

ConfigList list_for(int op, int dtype)
{
    if (op == TG_OP_GEMM) {
        if (dtype == TG_F32)
            return tg::configs_gemm_f32();
        if (dtype == TG_F16)
            return tg::configs_gemm_f16();
        if (dtype == TG_BF16)
            return tg::configs_gemm_bf16();
    } else if (op == TG_OP_DEQUANT_W4) {
        return tg::configs_dequant_w4();
    } else if (op == TG_OP_MX) {
        return tg::configs_mx();  // both activation formats
    } else if (op == TG_OP_SP24) {
        return tg::configs_sp24(dtype);
    }
    return ConfigList{nullptr, 0};
}

void config_name(const Config& c, char* buf, size_t len)
{
    static const char* dn[] = {"f32", "f16", "bf16"};
    static const char* mxn[] = {"e2m1", "e4m3"};
    static const char* lay[] = {"", "_nt", "_tn", "_tt"};  // A^T-stored / B^T-stored
    const bool mx = c.op == TG_OP_MX;
    static const char* opn[] = {"gemm", "w4", "mx", "sp24"};
    char wav[24];
    if (c.ks > 1)
        snprintf(wav, sizeof wav, "w%dx%dx%d", c.wgm, c.wgn, c.ks);  // k-slice groups last
    else
        snprintf(wav, sizeof wav, "w%dx%d", c.wgm, c.wgn);
    snprintf(buf, len, "%s_%s_%dx%dx%d_%s_s%d_g%d%s%s%s%s", opn[c.op],
             mx ? mxn[c.dtype] : dn[c.dtype], c.bm,
             c.bn, c.bk, wav, c.stages, c.group_m,
             c.pipe == 1 ? "_deep" : (c.pipe == 2 ? "_dma" : (c.pipe == 3 ? "_gemv" : "")),
             c.runs ? "_runs" : "",
             c.chunked_scales ? (mx ? (c.stages <= 3 ? "_sc4" : "_sc8")
                                    : (c.op == TG_OP_SP24 ? "_mc4" : (c.bk == 256 ? "_sc8" : "_sc16")))
                              : lay[(c.ta ? 2 : 0) + (c.tb ? 1 : 0)],
             c.wide ? "" : "_narrow");
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Elements per 16-byte chunk for the operand type.
int vec_of(int dtype) { return dtype == TG_F32 ? 4 : 8; }
int esize_of(int dtype) { return dtype == TG_F32 ? 4 : 2; }

int64_t tiles(int64_t x, int t) { return (x + t - 1) / t; }

const Config* find_by_name(int op, int dtype, const char* name);

// The weight-streaming dequant kernel for this K and scale alignment, or
// nullptr.  The variant with dword scale loads (bk == 128) needs K % 128 == 0
// and scale rows that start 4-byte aligned; the byte-load variant (bk == 32)
// takes any scale pointer.
// The row-run variant for calls of at least kGemvRunsMinM activation rows,
// whose activation loads bound the lane-range variant.
constexpr int64_t kGemvRunsMinM = 10;
const Config* gemv_for(int64_t M, int64_t K, bool ws4)
{
    ConfigList L = list_for(TG_OP_DEQUANT_W4, TG_BF16);
    const bool runs = M >= kGemvRunsMinM;
    for (int i = 0; i < L.count; ++i) {
        const Config& c = L.items[i];
        if (c.pipe == 3 && c.runs == runs && K % c.bk == 0 && (ws4 || c.bk != 128))
            return &c;
    }
    return nullptr;
}

// What a call needs from a configuration.
struct Call {
    int op, dtype;
    int64_t M, N, K;
    bool wide;    // 16-byte aligned operands whose rows are whole 16-byte chunks
    bool ws4;     // dequant / MX scale bytes start 4-byte aligned
    bool ta, tb;  // A stored [K][M], B stored [N][K]
    bool ws16 = false;  // MX scale / sparse metadata bytes start 16-byte aligned
};

// Whether configuration c can run call q.
bool usable(const Config& c, const Call& q)
{
    if (c.wide && !q.wide)
        return false;
    if (c.op == TG_OP_MX) {
        // activation format compiled in; whole 128-k strips; dword scale
        // copies, or 16-byte chunk copies that never straddle a row end
        if (c.chunked_scales && (q.K % 512 != 0 || !q.ws16))
            return false;
        if (c.bk == 256 && q.K % 1024 != 0)
            return false;  // 256-k strips: whole 4-strip scale chunks
        return c.dtype == q.dtype && q.wide && q.ws4 && q.K % c.bk == 0;
    }
    if (c.op == TG_OP_SP24) {
        // metadata chunks of 4 strips: whole 16-byte pieces of 16-byte aligned rows
        if (c.chunked_scales && (q.K % 256 != 0 || !q.ws16))
            return false;
        // whole 32-k groups of metadata dwords; 16-byte copies of values and B
        return c.dtype == q.dtype && q.wide && q.ws4 && q.K % 32 == 0;
    }
    if (c.ta != q.ta || c.tb != q.tb)
        return false;  // operand layouts are compiled in
    if (c.op == TG_OP_DEQUANT_W4 && (c.pipe == 2 || c.pipe == 3) && q.K % c.bk != 0)
        return false;  // whole strips / rounds of bk
    if (c.op == TG_OP_DEQUANT_W4 && (c.pipe == 2 || (c.pipe == 3 && c.bk == 128)) && !q.ws4)
        return false;  // scale bytes are copied / loaded as dwords
    if (c.op == TG_OP_DEQUANT_W4 && c.chunked_scales && (q.K % 512 != 0 || !q.ws16))
        return false;  // scale blocks: whole 16-byte pieces of 16-byte aligned rows
    return true;
}

// The names of every compiled configuration, per (op, dtype) list, formatted
// once: a call's selection looks names up in the tables above, and formatting
// every candidate's name per call took 5-20 us of host time.  (A function-local
// static is initialised once, thread-safely.)
const std::vector<std::string>& names_of(int op, int dtype)
{
    static const std::vector<std::vector<std::string>> tables = [] {
        std::vector<std::vector<std::string>> t(4 * 3);
        char buf[96];
        for (int o = 0; o < 4; ++o)
            for (int d = 0; d < 3; ++d) {
                ConfigList L = list_for(o, d);
                for (int i = 0; i < L.count; ++i) {
                    config_name(L.items[i], buf, sizeof buf);
                    t[o * 3 + d].push_back(buf);
                }
            }
        return t;
    }();
    static const std::vector<std::string> none;
    if (op < 0 || op >= 4 || dtype < 0 || dtype >= 3)
        return none;
    return tables[op * 3 + dtype];
}

const Config* find_by_name(int op, int dtype, const char* name)
{
    ConfigList L = list_for(op, dtype);
    const std::vector<std::string>& names = names_of(op, dtype);
    for (int i = 0; i < L.count && i < (int)names.size(); ++i)
        if (strcmp(names[i].c_str(), name) == 0)
            return &L.items[i];
    return nullptr;
}

// Compute units of the calling thread's current device, queried once per
// device (256 on MI355X; that value is also used when no device is visible,
// as for host-side configuration queries).
int64_t cu_count()
{
    static std::atomic<int> cache[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Rounds of tiles configuration c needs for an M x N output: one round is
// every compute unit running per_cu workgroups of it at once.
int64_t rounds(const Config& c, int64_t M, int64_t N, int per_cu)
{
    const int64_t slots = cu_count() * (per_cu > 0 ? per_cu : 1);
    return (tiles(M, c.bm) * tiles(N, c.bn) + slots - 1) / slots;
}

struct Choice {
    const Config* c;
    int group_m;  // 0: the configuration's default
};

// Fallback when the table holds nothing usable for a call (operand layouts
// and alignments the sweep does not time): the usable configuration whose
// last round of tiles leaves the least work per compute unit (rounds x tile
// area, one workgroup per unit), the larger tile on ties.
const Config* fallback(const Call& q)
{
    ConfigList L = list_for(q.op, q.dtype);
    const Config* best = nullptr;
    int64_t best_cost = 0;
    for (int i = 0; i < L.count; ++i) {
        const Config& c = L.items[i];
        if (!usable(c, q))
            continue;
        const int64_t cost = rounds(c, q.M, q.N, 1) * c.bm * c.bn;
        if (!best || cost < best_cost ||
            (cost == best_cost && c.bm * c.bn > best->bm * best->bn)) {
            best = &c;
            best_cost = cost;
        }
    }
    return best;
}

double lg2(int64_t x) { return log2((double)(x > 1 ? x : 1)); }

// The table, indexed once per process: exact entries and bucket
// representatives with their configurations resolved to list entries.
struct RepConfig {
    const Config* c;
    int group_m;
    double ms;
    int per_cu;
};
struct Rep {
    int op, dtype;
    int64_t M, N, K;
    double lm, ln, lk;  // log2 of M, N, K
    std::vector<RepConfig> configs;
};
struct ExactEntry {
    int op, dtype;
    int64_t M, N, K;
    const Config* c;
    int group_m;
};
struct TableIndex {
    std::vector<ExactEntry> exact;
    std::vector<Rep> reps;
};

const TableIndex& table_index()
{
    static const TableIndex idx = [] {
        TableIndex t;
        for (const TunedEntry& e : kTuned) {
            if (!e.config)
                continue;
            const Config* c = find_by_name(e.op, e.dtype, e.config);
            if (!c)
                continue;  // not compiled into this build
            if (e.exact) {
                t.exact.push_back({e.op, e.dtype, e.M, e.N, e.K, c, e.group_m});
                continue;
            }
            Rep* r = nullptr;
            for (Rep& x : t.reps)
                if (x.op == e.op && x.dtype == e.dtype && x.M == e.M && x.N == e.N && x.K == e.K)
                    r = &x;
            if (!r) {
                t.reps.push_back({e.op, e.dtype, e.M, e.N, e.K, lg2(e.M), lg2(e.N), lg2(e.K), {}});
                r = &t.reps.back();
            }
            r->configs.push_back({c, e.group_m, e.ms, e.per_cu});
        }
        return t;
    }();
    return idx;
}

// The selection: an exact table entry for the shape; else the bucket whose
// representative shape is nearest in log2(M), log2(N), log2(K), where each of
// its measured configurations is priced at the call's shape as
//   measured time x rounds(call) / rounds(representative) x K / K_rep
// (run time goes with the number of tile rounds and with K), and the cheapest
// usable one wins; else the fallback.  Few activation rows of the dequant
// GEMM take the weight-streaming kernel (its workgroups hold 16 rows).
Choice select_uncached(const Call& q)
{
    if (q.op == TG_OP_DEQUANT_W4 && q.M <= 16 && q.wide) {
        if (const Config* c = gemv_for(q.M, q.K, q.ws4))
            return {c, 0};
    }
    const TableIndex& t = table_index();
    for (const ExactEntry& e : t.exact) {
        if (e.op == q.op && e.dtype == q.dtype && e.M == q.M && e.N == q.N && e.K == q.K &&
            e.c->wide == q.wide && usable(*e.c, q))
            return {e.c, e.group_m};
    }
    const double lm = lg2(q.M), ln = lg2(q.N), lk = lg2(q.K);
    const Rep* rep = nullptr;
    double best_d = 0.0;
    for (const Rep& r : t.reps) {
        if (r.op != q.op || r.dtype != q.dtype)
            continue;
        const double d = fabs(lm - r.lm) + fabs(ln - r.ln) + fabs(lk - r.lk);
        if (!rep || d < best_d) {
            rep = &r;
            best_d = d;
        }
    }
    if (rep) {
        const RepConfig* best = nullptr;
        double best_est = 0.0;
        for (const RepConfig& rc : rep->configs) {
            if (!usable(*rc.c, q))
                continue;
            const double est = rc.ms * (double)rounds(*rc.c, q.M, q.N, rc.per_cu) /
                               (double)rounds(*rc.c, rep->M, rep->N, rc.per_cu) * (double)q.K /
                               (double)rep->K;
            if (!best || est < best_est) {
                best = &rc;
                best_est = est;
            }
        }
        if (best)
            return {best->c, best->group_m};
    }
    return {fallback(q), 0};
}

// select_uncached with a one-entry cache per thread: a loop that repeats one
// call pays the table search once.
Choice select_config(const Call& q)
{
    thread_local Call last{-1, -1, 0, 0, 0, false, false, false, false};
    thread_local Choice last_choice{nullptr, 0};
    thread_local int last_device = -1;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        (void)hipGetLastError();
    if (last.op == q.op && last.dtype == q.dtype && last.M == q.M && last.N == q.N &&
        last.K == q.K && last.wide == q.wide && last.ws4 == q.ws4 && last.ta == q.ta &&
        last.tb == q.tb && last.ws16 == q.ws16 && last_device == dev)
        return last_choice;
    last_choice = select_uncached(q);
    last = q;
    last_device = dev;
    return last_choice;
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

constexpr int64_t kMaxDim = 0x7FFFFFFF;

// Shape limits that keep every per-tile byte offset inside 31 bits.
tg_status check_shape(int64_t M, int64_t N, int64_t K, int esize)
{
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return TG_ERR_BAD_SHAPE;
    if (256 * K * esize > kMaxDim || 128 * N * esize > kMaxDim)
        return TG_ERR_BAD_SHAPE;
    if (tiles(M, 32) * tiles(N, 32) > kMaxDim)
        return TG_ERR_BAD_SHAPE;
    return TG_OK;
}

// Device buffer of the optional clock record (tg_set_clock_stamps), or NULL.
std::atomic<unsigned long long*> g_stamps{nullptr};
// Swizzle group forced on every launch by the tuning sweep (0: none).
std::atomic<int> g_group_override{0};

tg_status launch(const Config& c, const tg::GemmParams& base, hipStream_t stream,
                 int group_m = 0)
{
    tg::GemmParams p = base;
    p.stamps = g_stamps.load(std::memory_order_relaxed);
    const int forced_group = g_group_override.load(std::memory_order_relaxed);
    p.group_m = forced_group > 0 ? forced_group : group_m;
    p.tiles_m = (int)tiles(p.M, c.bm);
    p.tiles_n = (int)tiles(p.N, c.bn);
    const int64_t grid = (int64_t)p.tiles_m * p.tiles_n * (p.splits > 1 ? p.splits : 1);
    if (grid > kMaxDim)
        return TG_ERR_BAD_SHAPE;
    const char* fault = getenv("TG_FAULT");
    if (fault && strcmp(fault, "launch") == 0)
        return TG_ERR_HIP;  // forced failure, for testing error reporting
    if (getenv("TG_LOG")) {
        char name[96];
        config_name(c, name, sizeof name);
        fprintf(stderr, "[tilegemm] M=%d N=%d K=%d -> %s grid=%lld\n", p.M, p.N, p.K, name,
                (long long)grid);
    }
    void* args[] = {&p};
    hipError_t e = hipLaunchKernel(c.kernel, dim3((unsigned)grid), dim3(c.wgm * c.wgn * c.ks * 64), args,
                                   0, stream);
    // hipLaunchKernel's own status covers this launch; the thread's sticky
    // last-error state may hold an earlier call's error and is not consulted
    return e == hipSuccess ? TG_OK : TG_ERR_HIP;
}

// Split K (tg_gemm_splitk): the caller's request and workspace.
struct SplitArgs {
    int splits;  // 0: chosen by the library; >= 1: requested
    void* workspace;
    size_t bytes;
    bool use_scratch = false;  // tg_gemm_splitk_noalloc: the static scratch array
};

// How configuration c splits a call: S workgroups per tile over kc k each
// (whole strips), and the workspace bytes that takes (0 when S == 1).
struct SplitPlan {
    int S;
    int kc;
    size_t bytes;
};

constexpr size_t kCounterAlign = 256;

// Automatic split count: about one workgroup per compute unit, each split
// at least kMinSplitK k deep (1024 for 16-bit operands, 512 for fp32: shorter
// splits lose more to the pipeline fill and the partial-tile hand-off than
// the extra workgroups gain), and at most 16 partial tiles for the last
// workgroup to sum.  Measured on 256^2 x 8192, 128^2 x 16384, 512^2 x 8192 and
// 64 x 4096 x 4096 (bf16), 256^2 x 4096 and 512^3 (fp32).
constexpr int kMaxAutoSplits = 16;

SplitPlan split_plan(const Config& c, int64_t M, int64_t N, int64_t K, int splits)
{
    const int64_t t = tiles(M, c.bm) * tiles(N, c.bn);
    const int64_t strips = tiles(K, c.bk);
    int64_t S = splits;
    if (S <= 0) {
        const int64_t kmin = c.dtype == TG_F32 ? 512 : 1024;
        S = (256 + t - 1) / t;
        S = S < K / kmin ? S : K / kmin;
        S = S < kMaxAutoSplits ? S : kMaxAutoSplits;
    }
    if (S > strips)
        S = strips;
    if (S < 1)
        S = 1;
    const int64_t kc = ((strips + S - 1) / S) * c.bk;
    const int64_t used = K > 0 ? (K + kc - 1) / kc : 1;  // splits with work
    SplitPlan P{(int)used, (int)kc, 0};
    if (used > 1)
        P.bytes = ((size_t)t * 4 + kCounterAlign - 1) / kCounterAlign * kCounterAlign +
                  (size_t)t * (size_t)used * (size_t)c.bm * (size_t)c.bn * 4;
    return P;
}

// Configurations that can split K: the register-staged ones with k-slice
// wave groups (16-byte loads, plain layouts), larger tiles first.
int split_candidates(int dtype, const Config** out, int cap)
{
    ConfigList L = list_for(TG_OP_GEMM, dtype);
    int n = 0;
    for (int i = 0; i < L.count && n < cap; ++i)
        if (L.items[i].ks > 1 && L.items[i].wide && !L.items[i].ta && !L.items[i].tb)
            out[n++] = &L.items[i];
    for (int i = 1; i < n; ++i)  // insertion sort by tile area, descending
        for (int j = i; j > 0 && out[j]->bm * out[j]->bn > out[j - 1]->bm * out[j - 1]->bn; --j) {
            const Config* x = out[j];
            out[j] = out[j - 1];
            out[j - 1] = x;
        }
    return n;
}

// The split configuration: 64 x 64 tiles with two k-slice groups of 2 x 2
// waves for 16-bit operands, 32 x 32 tiles with four single-wave groups for
// fp32 (the fastest split configurations on the shapes above).
const Config* split_config(const Call& q)
{
    static const char* names[3] = {"gemm_f32_32x32x128_w1x1x4_s2_g8_deep",
                                   "gemm_f16_64x64x128_w2x2x2_s2_g8_deep",
                                   "gemm_bf16_64x64x128_w2x2x2_s2_g8_deep"};
    const Config* c = find_by_name(TG_OP_GEMM, q.dtype, names[q.dtype]);
    return c && usable(*c, q) ? c : nullptr;
}

tg_status gemm_impl(const Config* forced, int forced_index, int64_t M, int64_t N, int64_t K,
                    tg_dtype dtype, const void* A, int trans_a, const void* B, int trans_b,
                    void* C, tg_epilogue epi, tg_stream_t stream, const SplitArgs* sk = nullptr)
{
    if (dtype != TG_F32 && dtype != TG_F16 && dtype != TG_BF16)
        return TG_ERR_BAD_DTYPE;
    if (epi != TG_EPI_NONE && epi != TG_EPI_RELU)
        return TG_ERR_BAD_EPILOGUE;
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1))
        return TG_ERR_BAD_LAYOUT;
    const int es = esize_of(dtype);
    tg_status s = check_shape(M, N, K, es);
    if (s != TG_OK)
        return s;
    if (trans_a && 128 * M * es > kMaxDim)
        return TG_ERR_BAD_SHAPE;  // per-strip offsets of a [K][M] operand
    if (sk && sk->splits < 0)
        return TG_ERR_BAD_SHAPE;
    if (forced_index >= 0 && !forced)
        return TG_ERR_NO_CONFIG;
    if (sk && forced && forced->ks < 2)
        return TG_ERR_NO_CONFIG;  // only k-slice configurations split K
    if (M == 0 || N == 0)
        return TG_OK;
    // with K == 0 the operands hold no elements and are never read
    if (!C || (K > 0 && (!A || !B)))
        return TG_ERR_NULL_POINTER;
    const size_t cbytes = (size_t)(M * N * es);
    if (overlaps(C, cbytes, A, (size_t)(M * K * es)) || overlaps(C, cbytes, B, (size_t)(K * N * es)))
        return TG_ERR_ALIAS;
    if (sk && sk->workspace &&
        (overlaps(sk->workspace, sk->bytes, C, cbytes) ||
         overlaps(sk->workspace, sk->bytes, A, (size_t)(M * K * es)) ||
         overlaps(sk->workspace, sk->bytes, B, (size_t)(K * N * es))))
        return TG_ERR_ALIAS;
    const int v = vec_of(dtype);
    const int64_t lda = trans_a ? M : K, ldb = trans_b ? K : N;
    Call q{TG_OP_GEMM, dtype, M, N, K, false, false, trans_a != 0, trans_b != 0};
    // NULL is aligned
    q.wide = aligned16(A) && aligned16(B) && (lda % v == 0) && (ldb % v == 0);
    const Config* c = forced;
    int group_m = 0;
    SplitPlan plan{1, (int)K, 0};
    if (sk && (forced || q.wide)) {
        if (!c)
            c = split_config(q);
        if (c && usable(*c, q))
            plan = split_plan(*c, M, N, K, sk->splits);
        if (plan.S == 1 && !forced)
            c = nullptr;  // nothing to split: the plain selection below
    }
    if (!c) {
        const Choice ch = select_config(q);
        c = ch.c;
        group_m = ch.group_m;
    }
    if (!c || !usable(*c, q))
        return TG_ERR_NO_CONFIG;  // no (or a forced, unusable) configuration for this call
    void* ws = sk ? sk->workspace : nullptr;
    if (plan.S > 1 && sk->use_scratch) {
        if (plan.bytes > (size_t)TG_SPLITK_SCRATCH_BYTES)
            return TG_ERR_SCRATCH;
        if (scratch_of_device(&ws) != TG_OK)
            return TG_ERR_HIP;
    } else if (plan.S > 1 && (!ws || sk->bytes < plan.bytes || !aligned16(ws))) {
        return TG_ERR_WORKSPACE;
    }
    tg::GemmParams p{};
    if (plan.S > 1) {
        const int64_t t = tiles(M, c->bm) * tiles(N, c->bn);
        const size_t cnt = ((size_t)t * 4 + kCounterAlign - 1) / kCounterAlign * kCounterAlign;
        p.splits = plan.S;
        p.kc = plan.kc;
        p.counters = (int*)ws;
        p.ws = (float*)((char*)ws + cnt);
        if (sk->use_scratch) {
            // the array keeps the previous call's contents: its counters
            // must start at zero
            int* counters = p.counters;
            int n = (int)t;
            void* cargs[] = {&counters, &n};
            if (hipLaunchKernel((const void*)&tg_clear_counters, dim3((unsigned)((n + 255) / 256)),
                                dim3(256), cargs, 0, (hipStream_t)stream) != hipSuccess)
                return TG_ERR_HIP;
        }
    }
    p.A = A;
    p.B = B;
    p.Bs = nullptr;
    p.C = C;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.relu = epi == TG_EPI_RELU;
    p.c_vec = (N % 4 == 0) && ((uintptr_t)C % (dtype == TG_F32 ? 16 : 8) == 0);
    return launch(*c, p, (hipStream_t)stream, group_m);
}

tg_status w4_impl(const Config* forced, int forced_index, int64_t M, int64_t N, int64_t K,
                  const void* A, const uint8_t* Wq, const uint8_t* Ws, void* C, tg_epilogue epi,
                  tg_stream_t stream)
{
    if (epi != TG_EPI_NONE && epi != TG_EPI_RELU)
        return TG_ERR_BAD_EPILOGUE;
    tg_status s = check_shape(M, N, K, 2);
    if (s != TG_OK)
        return s;
    if (K % 32 != 0)
        return TG_ERR_BAD_SHAPE;
    if (forced_index >= 0 && !forced)
        return TG_ERR_NO_CONFIG;
    if (M == 0 || N == 0)
        return TG_OK;
    if (!C || (K > 0 && (!A || !Wq || !Ws)))
        return TG_ERR_NULL_POINTER;
    const size_t cbytes = (size_t)(M * N * 2);
    if (overlaps(C, cbytes, A, (size_t)(M * K * 2)) || overlaps(C, cbytes, Wq, (size_t)(N * K / 2)) ||
        overlaps(C, cbytes, Ws, (size_t)(N * K / 32)))
        return TG_ERR_ALIAS;
    Call q{TG_OP_DEQUANT_W4, TG_BF16, M, N, K, aligned16(A) && aligned16(Wq),
           ((uintptr_t)Ws & 3u) == 0, false, false};
    q.ws16 = aligned16(Ws);
    const Choice ch = forced ? Choice{forced, 0} : select_config(q);
    const Config* c = ch.c;
    if (!c || !usable(*c, q))
        return TG_ERR_NO_CONFIG;  // no (or a forced, unusable) configuration for this call
    tg::GemmParams p{};
    p.A = A;
    p.B = Wq;
    p.Bs = Ws;
    p.C = C;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.relu = epi == TG_EPI_RELU;
    p.c_vec = (N % 4 == 0) && ((uintptr_t)C % 8 == 0);
    return launch(*c, p, (hipStream_t)stream, ch.group_m);
}

tg_status mx_impl(const Config* forced, int forced_index, int64_t M, int64_t N, int64_t K,
                  int a_fmt, const uint8_t* Aq, const uint8_t* As, const uint8_t* Wq,
                  const uint8_t* Ws, void* C, tg_epilogue epi, tg_stream_t stream)
{
    if (a_fmt != TG_MX_E2M1 && a_fmt != TG_MX_E4M3)
        return TG_ERR_BAD_DTYPE;
    if (epi != TG_EPI_NONE && epi != TG_EPI_RELU)
        return TG_ERR_BAD_EPILOGUE;
    tg_status s = check_shape(M, N, K, 1);
    if (s != TG_OK)
        return s;
    if (K % 128 != 0)
        return TG_ERR_BAD_SHAPE;
    if (forced_index >= 0 && !forced)
        return TG_ERR_NO_CONFIG;
    if (M == 0 || N == 0)
        return TG_OK;
    if (!C || (K > 0 && (!Aq || !As || !Wq || !Ws)))
        return TG_ERR_NULL_POINTER;
    const size_t cbytes = (size_t)(M * N * 2);
    const size_t abytes = (size_t)(a_fmt == TG_MX_E4M3 ? M * K : M * K / 2);
    if (overlaps(C, cbytes, Aq, abytes) || overlaps(C, cbytes, As, (size_t)(M * K / 32)) ||
        overlaps(C, cbytes, Wq, (size_t)(N * K / 2)) || overlaps(C, cbytes, Ws, (size_t)(N * K / 32)))
        return TG_ERR_ALIAS;
    Call q{TG_OP_MX, a_fmt, M, N, K, aligned16(Aq) && aligned16(Wq),
           (((uintptr_t)As | (uintptr_t)Ws) & 3u) == 0, false, false};
    q.ws16 = aligned16(As) && aligned16(Ws);
    const Choice ch = forced ? Choice{forced, 0} : select_config(q);
    const Config* c = ch.c;
    if (!c || !usable(*c, q))
        return TG_ERR_NO_CONFIG;  // no (or a forced, unusable) configuration for this call
    tg::GemmParams p{};
    p.A = Aq;
    p.As = As;
    p.B = Wq;
    p.Bs = Ws;
    p.C = C;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.relu = epi == TG_EPI_RELU;
    p.c_vec = (N % 4 == 0) && ((uintptr_t)C % 8 == 0);
    return launch(*c, p, (hipStream_t)stream, ch.group_m);
}

tg_status sp24_impl(const Config* forced, int forced_index, int64_t M, int64_t N, int64_t K,
                    tg_dtype dtype, const void* Ac, const uint8_t* Ai, const void* B, void* C,
                    tg_epilogue epi, tg_stream_t stream)
{
    if (dtype != TG_F16 && dtype != TG_BF16)
        return TG_ERR_BAD_DTYPE;
    if (epi != TG_EPI_NONE && epi != TG_EPI_RELU)
        return TG_ERR_BAD_EPILOGUE;
    tg_status s = check_shape(M, N, K, 2);
    if (s != TG_OK)
        return s;
    if (K % 32 != 0)
        return TG_ERR_BAD_SHAPE;
    if (forced_index >= 0 && !forced)
        return TG_ERR_NO_CONFIG;
    if (M == 0 || N == 0)
        return TG_OK;
    if (!C || (K > 0 && (!Ac || !Ai || !B)))
        return TG_ERR_NULL_POINTER;
    const size_t cbytes = (size_t)(M * N * 2);
    if (overlaps(C, cbytes, Ac, (size_t)(M * K)) || overlaps(C, cbytes, Ai, (size_t)(M * K / 8)) ||
        overlaps(C, cbytes, B, (size_t)(K * N * 2)))
        return TG_ERR_ALIAS;
    Call q{TG_OP_SP24, dtype, M, N, K, aligned16(Ac) && aligned16(B) && N % 8 == 0,
           ((uintptr_t)Ai & 3u) == 0, false, false};
    q.ws16 = aligned16(Ai);
    const Choice ch = forced ? Choice{forced, 0} : select_config(q);
    const Config* c = ch.c;
    if (!c || !usable(*c, q))
        return TG_ERR_NO_CONFIG;  // no (or a forced, unusable) configuration for this call
    tg::GemmParams p{};
    p.A = Ac;
    p.As = Ai;
    p.B = B;
    p.C = C;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.relu = epi == TG_EPI_RELU;
    p.c_vec = 0;
    return launch(*c, p, (hipStream_t)stream, ch.group_m);
}

}  // namespace

extern "C" {

tg_status tg_gemm(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void* A, const void* B,
                  void* C, tg_epilogue epi, tg_stream_t stream)
{
    return gemm_impl(nullptr, -1, M, N, K, dtype, A, 0, B, 0, C, epi, stream);
}

tg_status tg_gemm_ex(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void* A, int trans_a,
                     const void* B, int trans_b, void* C, tg_epilogue epi, tg_stream_t stream)
{
    return gemm_impl(nullptr, -1, M, N, K, dtype, A, trans_a, B, trans_b, C, epi, stream);
}

tg_status tg_gemm_splitk_workspace_size(int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                        int splits, size_t* bytes)
{
    if (!bytes)
        return TG_ERR_NULL_POINTER;
    *bytes = 0;
    if (dtype != TG_F32 && dtype != TG_F16 && dtype != TG_BF16)
        return TG_ERR_BAD_DTYPE;
    tg_status s = check_shape(M, N, K, esize_of(dtype));
    if (s != TG_OK)
        return s;
    if (splits < 0)
        return TG_ERR_BAD_SHAPE;
    if (M == 0 || N == 0)
        return TG_OK;
    // enough for every split configuration, so forced configurations fit too
    const Config* cand[16];
    const int n = split_candidates(dtype, cand, 16);
    for (int i = 0; i < n; ++i) {
        const SplitPlan P = split_plan(*cand[i], M, N, K, splits);
        if (P.bytes > *bytes)
            *bytes = P.bytes;
    }
    return TG_OK;
}

tg_status tg_gemm_splitk(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void* A,
                         const void* B, void* C, tg_epilogue epi, int splits, void* workspace,
                         size_t workspace_bytes, tg_stream_t stream)
{
    const SplitArgs sk{splits, workspace, workspace_bytes};
    return gemm_impl(nullptr, -1, M, N, K, dtype, A, 0, B, 0, C, epi, stream, &sk);
}

tg_status tg_gemm_splitk_noalloc(int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                 const void* A, const void* B, void* C, tg_epilogue epi,
                                 int splits, tg_stream_t stream)
{
    SplitArgs sk{splits, nullptr, 0};
    sk.use_scratch = true;
    return gemm_impl(nullptr, -1, M, N, K, dtype, A, 0, B, 0, C, epi, stream, &sk);
}

tg_status tg_gemm_splitk_config(int index, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                const void* A, const void* B, void* C, tg_epilogue epi,
                                int splits, void* workspace, size_t workspace_bytes,
                                tg_stream_t stream)
{
    if (dtype != TG_F32 && dtype != TG_F16 && dtype != TG_BF16)
        return TG_ERR_BAD_DTYPE;
    ConfigList L = list_for(TG_OP_GEMM, dtype);
    const Config* c = (index >= 0 && index < L.count) ? &L.items[index] : nullptr;
    const SplitArgs sk{splits, workspace, workspace_bytes};
    return gemm_impl(c, index < 0 ? 0 : index, M, N, K, dtype, A, 0, B, 0, C, epi, stream, &sk);
}

tg_status tg_dequant_gemm_w4(int64_t M, int64_t N, int64_t K, const void* A, const uint8_t* Wq,
                             const uint8_t* Ws, void* C, tg_epilogue epi, tg_stream_t stream)
{
    return w4_impl(nullptr, -1, M, N, K, A, Wq, Ws, C, epi, stream);
}

tg_status tg_gemm_mx(int64_t M, int64_t N, int64_t K, tg_mx_format a_fmt, const uint8_t* Aq,
                     const uint8_t* As, const uint8_t* Wq, const uint8_t* Ws, void* C,
                     tg_epilogue epi, tg_stream_t stream)
{
    return mx_impl(nullptr, -1, M, N, K, a_fmt, Aq, As, Wq, Ws, C, epi, stream);
}

tg_status tg_gemm_sp24(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void* Ac,
                       const uint8_t* Ai, const void* B, void* C, tg_epilogue epi,
                       tg_stream_t stream)
{
    return sp24_impl(nullptr, -1, M, N, K, dtype, Ac, Ai, B, C, epi, stream);
}

const char* tg_status_str(tg_status s)
{
    switch (s) {
    case TG_OK:
        return "TG_OK: success";
    case TG_ERR_NULL_POINTER:
        return "TG_ERR_NULL_POINTER: a required pointer is NULL";
    case TG_ERR_BAD_SHAPE:
        return "TG_ERR_BAD_SHAPE: negative or too large size, or K not a multiple of 32 (dequant) "
               "or 128 (MX)";
    case TG_ERR_BAD_DTYPE:
        return "TG_ERR_BAD_DTYPE: dtype must be TG_F32, TG_F16 or TG_BF16 (MX: TG_MX_E2M1 or "
               "TG_MX_E4M3)";
    case TG_ERR_BAD_EPILOGUE:
        return "TG_ERR_BAD_EPILOGUE: epilogue must be TG_EPI_NONE or TG_EPI_RELU";
    case TG_ERR_ALIAS:
        return "TG_ERR_ALIAS: the output overlaps an input";
    case TG_ERR_NO_CONFIG:
        return "TG_ERR_NO_CONFIG: no such kernel configuration for this call";
    case TG_ERR_HIP:
        return "TG_ERR_HIP: the HIP runtime reported an error at launch";
    case TG_ERR_BAD_LAYOUT:
        return "TG_ERR_BAD_LAYOUT: trans_a and trans_b must be 0 or 1";
    case TG_ERR_WORKSPACE:
        return "TG_ERR_WORKSPACE: split-K workspace NULL, smaller than "
               "tg_gemm_splitk_workspace_size, or not 16-byte aligned";
    case TG_ERR_SCRATCH:
        return "TG_ERR_SCRATCH: the split needs more than the fixed scratch array "
               "(TG_SPLITK_SCRATCH_BYTES); use tg_gemm_splitk with a workspace, or fewer splits";
    }
    return "unknown tg_status";
}

tg_status tg_query_config_ex(int op, int64_t M, int64_t N, int64_t K, tg_dtype dtype, int trans_a,
                             int trans_b, char* buf, size_t len)
{
    if (!buf || len == 0)
        return TG_ERR_NULL_POINTER;
    if (op != TG_OP_GEMM && op != TG_OP_DEQUANT_W4 && op != TG_OP_MX && op != TG_OP_SP24)
        return TG_ERR_NO_CONFIG;
    if (op == TG_OP_SP24 && dtype != TG_F16 && dtype != TG_BF16)
        return TG_ERR_BAD_DTYPE;
    if (op == TG_OP_GEMM && dtype != TG_F32 && dtype != TG_F16 && dtype != TG_BF16)
        return TG_ERR_BAD_DTYPE;
    if (op == TG_OP_MX && (int)dtype != TG_MX_E2M1 && (int)dtype != TG_MX_E4M3)
        return TG_ERR_BAD_DTYPE;  // the activation format
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1) ||
        (op != TG_OP_GEMM && (trans_a || trans_b)))
        return TG_ERR_BAD_LAYOUT;
    const int dt = op == TG_OP_DEQUANT_W4 ? TG_BF16 : dtype;
    tg_status s = check_shape(M, N, K, op == TG_OP_MX ? 1 : esize_of(dt));
    if (s != TG_OK)
        return s;
    if ((op == TG_OP_DEQUANT_W4 && K % 32 != 0) || (op == TG_OP_MX && K % 128 != 0) ||
        (op == TG_OP_SP24 && K % 32 != 0))
        return TG_ERR_BAD_SHAPE;
    // assume aligned operands (what torch allocations give)
    const int64_t lda = trans_a ? M : K, ldb = trans_b ? K : N;
    Call q{op, dt, M, N, K, false, true, trans_a != 0, trans_b != 0};
    q.ws16 = true;
    q.wide = op == TG_OP_SP24 ? N % 8 == 0
                              : (op != TG_OP_GEMM || (lda % vec_of(dt) == 0 && ldb % vec_of(dt) == 0));
    const Choice ch = select_config(q);
    const Config* c = ch.c;
    if (!c)
        return TG_ERR_NO_CONFIG;
    char name[96];
    config_name(*c, name, sizeof name);
    snprintf(buf, len, "%s grid=%lld threads=%d group=%d", name,
             (long long)(tiles(M, c->bm) * tiles(N, c->bn)), c->wgm * c->wgn * c->ks * 64,
             ch.group_m > 0 ? ch.group_m : c->group_m);
    return TG_OK;
}

tg_status tg_query_config(int op, int64_t M, int64_t N, int64_t K, tg_dtype dtype, char* buf,
                          size_t len)
{
    return tg_query_config_ex(op, M, N, K, dtype, 0, 0, buf, len);
}

int tg_config_count(int op, tg_dtype dtype)
{
    return list_for(op, op == TG_OP_DEQUANT_W4 ? TG_BF16 : dtype).count;
}

tg_status tg_config_name(int op, tg_dtype dtype, int index, char* buf, size_t len)
{
    if (!buf || len == 0)
        return TG_ERR_NULL_POINTER;
    ConfigList L = list_for(op, op == TG_OP_DEQUANT_W4 ? TG_BF16 : dtype);
    if (index < 0 || index >= L.count)
        return TG_ERR_NO_CONFIG;
    config_name(L.items[index], buf, len);
    return TG_OK;
}

tg_status tg_gemm_config(int index, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                         const void* A, const void* B, void* C, tg_epilogue epi,
                         tg_stream_t stream)
{
    if (dtype != TG_F32 && dtype != TG_F16 && dtype != TG_BF16)
        return TG_ERR_BAD_DTYPE;
    ConfigList L = list_for(TG_OP_GEMM, dtype);
    const Config* c = (index >= 0 && index < L.count) ? &L.items[index] : nullptr;
    return gemm_impl(c, index < 0 ? 0 : index, M, N, K, dtype, A, 0, B, 0, C, epi, stream);
}

tg_status tg_gemm_ex_config(int index, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                            const void* A, int trans_a, const void* B, int trans_b, void* C,
                            tg_epilogue epi, tg_stream_t stream)
{
    if (dtype != TG_F32 && dtype != TG_F16 && dtype != TG_BF16)
        return TG_ERR_BAD_DTYPE;
    ConfigList L = list_for(TG_OP_GEMM, dtype);
    const Config* c = (index >= 0 && index < L.count) ? &L.items[index] : nullptr;
    return gemm_impl(c, index < 0 ? 0 : index, M, N, K, dtype, A, trans_a, B, trans_b, C, epi,
                     stream);
}

tg_status tg_dequant_gemm_w4_config(int index, int64_t M, int64_t N, int64_t K, const void* A,
                                    const uint8_t* Wq, const uint8_t* Ws, void* C,
                                    tg_epilogue epi, tg_stream_t stream)
{
    ConfigList L = list_for(TG_OP_DEQUANT_W4, TG_BF16);
    const Config* c = (index >= 0 && index < L.count) ? &L.items[index] : nullptr;
    return w4_impl(c, index < 0 ? 0 : index, M, N, K, A, Wq, Ws, C, epi, stream);
}

tg_status tg_gemm_mx_config(int index, int64_t M, int64_t N, int64_t K, tg_mx_format a_fmt,
                            const uint8_t* Aq, const uint8_t* As, const uint8_t* Wq,
                            const uint8_t* Ws, void* C, tg_epilogue epi, tg_stream_t stream)
{
    ConfigList L = list_for(TG_OP_MX, 0);
    const Config* c = (index >= 0 && index < L.count) ? &L.items[index] : nullptr;
    return mx_impl(c, index < 0 ? 0 : index, M, N, K, a_fmt, Aq, As, Wq, Ws, C, epi, stream);
}

tg_status tg_gemm_sp24_config(int index, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                              const void* Ac, const uint8_t* Ai, const void* B, void* C,
                              tg_epilogue epi, tg_stream_t stream)
{
    if (dtype != TG_F16 && dtype != TG_BF16)
        return TG_ERR_BAD_DTYPE;
    ConfigList L = list_for(TG_OP_SP24, dtype);
    const Config* c = (index >= 0 && index < L.count) ? &L.items[index] : nullptr;
    return sp24_impl(c, index < 0 ? 0 : index, M, N, K, dtype, Ac, Ai, B, C, epi, stream);
}

void tg_set_clock_stamps(uint64_t* stamps)
{
    g_stamps.store((unsigned long long*)stamps, std::memory_order_relaxed);
}

void tg_set_swizzle_override(int group_m)
{
    g_group_override.store(group_m > 0 ? group_m : 0, std::memory_order_relaxed);
}

tg_status tg_config_occupancy(int op, tg_dtype dtype, int index, int* workgroups_per_cu)
{
    if (!workgroups_per_cu)
        return TG_ERR_NULL_POINTER;
    *workgroups_per_cu = 0;
    ConfigList L = list_for(op, op == TG_OP_DEQUANT_W4 ? TG_BF16 : dtype);
    if (index < 0 || index >= L.count)
        return TG_ERR_NO_CONFIG;
    const Config& c = L.items[index];
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, c.kernel, c.wgm * c.wgn * c.ks * 64, 0) !=
        hipSuccess)
        return TG_ERR_HIP;
    *workgroups_per_cu = n;
    return TG_OK;
}

tg_status tg_tile_map(int64_t tiles_m, int64_t tiles_n, int group_m, int32_t* out_m,
                      int32_t* out_n)
{
    if (!out_m || !out_n)
        return TG_ERR_NULL_POINTER;
    if (tiles_m < 1 || tiles_n < 1 || group_m < 1 || tiles_m * tiles_n > kMaxDim)
        return TG_ERR_BAD_SHAPE;
    const int total = (int)(tiles_m * tiles_n);
    for (int w = 0; w < total; ++w) {
        tg::TileCoord t = tg::tile_of(w, (int)tiles_m, (int)tiles_n, group_m);
        out_m[w] = t.m;
        out_n[w] = t.n;
    }
    return TG_OK;
}

}  // extern "C"
