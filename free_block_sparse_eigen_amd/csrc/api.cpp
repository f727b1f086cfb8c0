// C ABI of the SparsePR attention-call hot path: validation, workspace, stage
// sequencing, host fp64 solves and launches. See include/sparsepr.h for the contract.
#include "../../include/sparsepr.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstdio>
#include <cstring>
#include <functional>
#include <memory>
#include <mutex>
#include <numeric>
#include <string>
#include <thread>
#include <vector>

#include "host_linalg.h"
#include "kernels.h"

using namespace spr;

namespace {

// Host worker threads kept for the life of a context (starting threads per call costs
// more than the per-head work they run). run() hands tasks 0..n-1 out through an atomic
// counter to the workers and the calling thread, and returns when all have finished.
class HostPool {
public:
    explicit HostPool(int workers) {
        for (int i = 0; i < workers; ++i) th_.emplace_back([this] { loop(); });
    }
    ~HostPool() {
        {
            std::lock_guard<std::mutex> g(m_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& t : th_) t.join();
    }
    void run(int tasks, const std::function<void(int)>& fn) {
        {
            std::lock_guard<std::mutex> g(m_);
            job_ = &fn;
            ntasks_ = tasks;
            next_.store(0);
            ++gen_;
        }
        cv_.notify_all();
        drain();
        std::unique_lock<std::mutex> lk(m_);
        done_.wait(lk, [&] { return active_ == 0 && next_.load() >= ntasks_; });
    }

private:
    void drain() {
        for (int t; (t = next_.fetch_add(1)) < ntasks_;) (*job_)(t);
    }
    void loop() {
        unsigned seen = 0;
        std::unique_lock<std::mutex> lk(m_);
        for (;;) {
            cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
            if (stop_) return;
            seen = gen_;
            ++active_;
            lk.unlock();
            drain();
            lk.lock();
            if (--active_ == 0) done_.notify_all();
        }
    }
    std::mutex m_;
    std::condition_variable cv_, done_;
    std::vector<std::thread> th_;
    const std::function<void(int)>* job_ = nullptr;
    int ntasks_ = 0;
    std::atomic<int> next_{0};
    int active_ = 0;
    unsigned gen_ = 0;
    bool stop_ = false;
};

}  // namespace

// Streams the partition's heads are spread over (one group of consecutive heads each).
constexpr int kPartitionStreams = 2;
constexpr int64_t kBigUnitsMinRows = int64_t(1) << 17;   // H N from which 256-row units run

struct sparsepr_ctx {
    sparsepr_params p{};
    int device = 0;
    int H = 0, N = 0, d = 0, Gk = 0, Gq = 0, rK = 0, Dq = 0, k = 0, P = 0, T = 0;
    int nblk = 0, maxu = 0, maxu_big = 0, splits = 0, dense_units = 0, gmax = 0;
    bool big_units = false;            // whole 256-row chunks of a query group as 8-wave units
    bool raw = false;                  // SPARSEPR_F_RAW_KMEANS: identity metrics on both sides
    bool svoo = false;                 // SPARSEPR_F_SVOO: alternating co-clustering
    bool fp8 = false;                  // SPARSEPR_F_FP8_QK: fp8 logits in the sparse kernel
    bool have_route = false;           // a partition and routing exist (sparsepr_reuse_route)
    int64_t weyl_a = 0;

    void* arena = nullptr;
    size_t arena_bytes = 0;
    // bf16 copies of fp32 inputs, and the group-major K/V
    bf16_t *qb = nullptr, *kb = nullptr, *vb = nullptr;
    bf16_t* kp = nullptr;                         // K in group-major order
    uint16_t* vp = nullptr;                       // V in group-major order, fp16 scaled per head
    uint32_t* vmax = nullptr;                     // [H] largest |v| per head (bf16 magnitude bits)
    // SPARSEPR_F_FP8_QK (an experiment): K group-major in FP8 E4M3, per-head largest |q|, |k|
    uint8_t* kp8 = nullptr;
    uint32_t *qmax = nullptr, *kmax = nullptr;
    unsigned long long* nonfinite = nullptr;      // [2] non-finite inputs, outputs (CHECK_FINITE)
    const bf16_t* q_src = nullptr;                // Q in token order (the route stage's input)
    const bf16_t* v_src = nullptr;                // V in token order (the probe rows gather it)
    // partition
    int32_t *klab = nullptr, *qlab = nullptr, *kperm = nullptr, *qperm = nullptr;
    int32_t *koff = nullptr, *qoff = nullptr;
    int32_t *flag_cnt = nullptr, *flag_list = nullptr, *blkhist = nullptr, *blkoff = nullptr;
    // candidate lists of the recheck queue (full metric, streamed centroids: large G)
    int32_t *cand = nullptr, *ncand = nullptr, *ovf_cnt = nullptr, *ovf_list = nullptr;
    double* crow = nullptr;            // [H][G][d] row-major screening vectors / coordinates
    double* ycoord = nullptr;          // [H][N][r_K] every key's coordinates x W (candidate recheck)
    bf16_t* zhl = nullptr;             // [H][N][2][r_K] the same split in bf16 hi, lo (key screen)
    float* zkb = nullptr;              // [H][N] each key's screen bound coefficient
    double *mk = nullptr, *w64 = nullptr, *kc64 = nullptr, *qc64 = nullptr;
    // device eigensolve of M_K: tridiagonal form, reflectors, eigenpairs, |T|, gap
    double *eig_diag = nullptr, *eig_off = nullptr, *eig_hv = nullptr, *eig_beta = nullptr;
    double *eig_lam = nullptr, *eig_vec = nullptr, *eig_tnorm = nullptr, *mgap = nullptr;
    bool dev_eig = false;              // M_K eigensolve on the device (else on the host)
    bool mgap_dev = false;             // the last partition's metric gaps are in mgap
    double* ident = nullptr;           // [H][d][d] identity metric (SPARSEPR_F_RAW_KMEANS)
    double *kc2 = nullptr, *qc2 = nullptr;               // fp64 |c|^2 per centroid
    double *kraw = nullptr, *qraw = nullptr;
    double* kraw_t = nullptr;          // [H][d][G_k] coordinate-major key centroids (routing)
    bf16_t *kcp = nullptr, *qcp = nullptr;               // screening vectors, bf16 hi/lo
    float *kcn2 = nullptr, *qcn2 = nullptr, *kcpn = nullptr, *qcpn = nullptr;
    // route
    int32_t *blocks = nullptr, *ucount = nullptr, *probe_pos = nullptr, *probe_orig = nullptr;
    int32_t *probe_grp = nullptr, *probe_of = nullptr, *nunits = nullptr, *nunits_big = nullptr;
    int2 *units = nullptr, *units_big = nullptr;
    int64_t* pairs = nullptr;
    // attention, probes, fit
    float *o_s = nullptr, *part_ml = nullptr, *part_od = nullptr, *part_os = nullptr;
    float *px = nullptr, *py = nullptr, *pod = nullptr, *bv32 = nullptr;
    bf16_t* bt16 = nullptr;                      // [H][2][d][d] B'^T as bf16 hi, lo
    double *fit_m = nullptr, *fit_g = nullptr;   // [H][2][d] means, [H][3][d][d] Grams
    double* mq = nullptr;                        // [H][d][d] query metric C_K^T C_K / d
    // dense baseline: one query group and one key group holding every token
    int32_t *dense_meta = nullptr;     // qoff {0,N}, koff {0,N}, blocks {0}, nunits {..}
    int2* dense_unit_list = nullptr;

    // host mirrors
    std::vector<double> h_bm, h_bv;
    std::vector<double> h_mgap, h_rgap;          // per-head spectral gaps of the last call
    std::vector<float> h_x, h_y;
    // pinned host buffers of the fit: Grams in (device -> host), B' and b' out
    double* h_fit = nullptr;          // [H][2][d] means, then [H][3][d][d] Grams
    double* h_mkp = nullptr;          // [H][d][d] M_K (device -> host)
    double* h_wp = nullptr;           // [H][d][r_K] key projection W (host -> device)
    void* h_b32 = nullptr;            // [H][2][d][d] bf16 B'^T hi/lo, then [H][d] fp32 b'
    hipEvent_t ev_probe = nullptr;    // probe rows and fit Grams are on the host
    hipEvent_t ev_rows = nullptr;     // probe rows merged (the fit's inputs are ready)
    hipEvent_t ev_kdone = nullptr;    // key partition done (the side stream may permute K)
    hipEvent_t ev_kperm = nullptr;    // K permuted on the side stream
    hipEvent_t ev_qside = nullptr;    // SPARSEPR_F_FP8_QK: the side stream may read q
    bool kperm_recorded = false;      // ev_kperm has been recorded
    hipStream_t side = nullptr;       // fit means, Grams and their copy to the host
    // the sparse kernel's 128-row units run on ustream beside the 256-row units (big_units)
    hipStream_t ustream = nullptr;
    hipEvent_t ev_ufork = nullptr, ev_ujoin = nullptr;
    // the partition's heads in nparts groups, group 0 on the caller's stream, group i > 0 on
    // pstream[i]
    static constexpr int kMaxParts = 4;
    int nparts = 1;
    hipStream_t pstream[kMaxParts] = {};
    hipEvent_t ev_fork = nullptr;               // the other groups may start
    hipEvent_t ev_kd[kMaxParts] = {};           // group i's keys are partitioned ([0]: ev_kdone)
    hipEvent_t ev_jn[kMaxParts] = {};           // group i is done
    // sparsepr_attention hands V to the partition stage (bf16 only), which takes its per-head
    // magnitudes on the side stream beside the eigensolve and permutes it there right after
    // K; the route stage skips its own V permute for that V
    const bf16_t* v_pre = nullptr;
    bool v_pre_done = false;

    int stage = 0;
    bool poisoned = false;
    std::string err;
    hipStream_t last_stream = nullptr;
    bool timing = false;
    bool check_finite = false;
    static constexpr int kRing = 64;   // per-call stage events kept for averaging
    hipEvent_t ev[kRing][8] = {};
    bool ev_used[kRing][8] = {};
    int64_t calls = 0;
    int64_t stats_from = 0;            // first call averaged by the next sparsepr_get_stats
    int slot = 0;
    std::unique_ptr<HostPool> pool;    // host workers for per-head work (made on first use)
};

namespace {

constexpr int kStagePartition = 1, kStageRoute = 2, kStageAttn = 3, kStageFit = 4, kStageCorrect = 5;

int64_t weyl_multiplier(int64_t n) {
    int64_t a = static_cast<int64_t>((static_cast<uint64_t>(n) * 0x9E3779B9ull) >> 32);
    while (std::gcd(a, n) != 1) ++a;
    return a;
}

int routed_count(double density, int gk) {
    int k = static_cast<int>(std::ceil(density * gk - 1e-9));
    return std::min(std::max(k, 1), gk);
}

int32_t validate(const sparsepr_params* p) {
    if (!p) return SPARSEPR_ERR_INVALID_ARG;
    if (p->heads < 1 || p->n < 1 || p->n > (1 << 24)) return SPARSEPR_ERR_SHAPE;
    if ((p->d == 64 || p->d == 128) && (int64_t)p->n * p->d * 2 >= ((int64_t)1 << 31))
        return SPARSEPR_ERR_SHAPE;                  // one head's rows past 32-bit buffer offsets
    if ((int64_t)p->heads * p->n > 0x7fffffffLL) return SPARSEPR_ERR_SHAPE;
    if (p->d != 64 && p->d != 128) return SPARSEPR_ERR_SHAPE;
    if (p->dtype != SPARSEPR_BF16 && p->dtype != SPARSEPR_F32) return SPARSEPR_ERR_INVALID_ARG;
    if (p->n_sample < 1 || p->n_sample > p->n) return SPARSEPR_ERR_INVALID_ARG;
    if (p->key_rank < 1 || p->key_rank > p->d) return SPARSEPR_ERR_INVALID_ARG;
    const int gmax = std::min(p->n, kMaxGroups);
    if (p->kv_groups < 1 || p->kv_groups > gmax) return SPARSEPR_ERR_INVALID_ARG;
    if (p->q_groups < 1 || p->q_groups > gmax) return SPARSEPR_ERR_INVALID_ARG;
    if (p->kmeans_iters < 1 || p->kmeans_iters > 100) return SPARSEPR_ERR_INVALID_ARG;
    if (p->probes < 0 || p->probes > std::min(p->n, 4096)) return SPARSEPR_ERR_INVALID_ARG;
    if (p->corr_rank < 0 || p->corr_rank > p->d) return SPARSEPR_ERR_INVALID_ARG;
    if (!(p->density > 0.0) || !(p->density <= 1.0)) return SPARSEPR_ERR_INVALID_ARG;
    if (!(p->ridge_lambda >= 0.0) || !std::isfinite(p->ridge_lambda)) return SPARSEPR_ERR_INVALID_ARG;
    if (p->flags & ~(SPARSEPR_F_STAGE_TIMING | SPARSEPR_F_RAW_KMEANS | SPARSEPR_F_CHECK_FINITE |
                     SPARSEPR_F_HOST_SOLVE | SPARSEPR_F_SVOO | SPARSEPR_F_SERIAL_PARTITION |
                     SPARSEPR_F_FP8_QK | SPARSEPR_F_RAW_KEY_SCREEN | SPARSEPR_F_UNIFORM_UNITS))
        return SPARSEPR_ERR_INVALID_ARG;
    if ((p->flags & SPARSEPR_F_RAW_KMEANS) && (p->flags & SPARSEPR_F_SVOO)) return SPARSEPR_ERR_INVALID_ARG;
    return SPARSEPR_OK;
}

// Arena layout: every buffer 256-byte aligned; pass 1 sizes, pass 2 assigns.
struct Arena {
    char* base = nullptr;
    size_t used = 0;
    template <typename T>
    void take(T*& ptr, size_t count) {
        used = (used + 255) & ~size_t(255);
        ptr = base ? reinterpret_cast<T*>(base + used) : nullptr;
        used += sizeof(T) * std::max<size_t>(count, 1);
    }
};

// The key side screens in its coordinates x W (bf16 hi + lo, depth 4 r_K instead of 2 d)
// when the centroids' split coordinates stay resident in LDS (G_k r_K of them, hi and lo)
// and r_K has a kernel (16 or 32): the W metric path only (not the identity-metric or
// co-clustering partitioners). Where the raw screen would stream its centroids (large G_k),
// the queued keys' candidate lists are screened in the same coordinates.
bool key_screen_in_coords(const sparsepr_ctx& c) {
    return !c.raw && !c.svoo && !(c.p.flags & SPARSEPR_F_RAW_KEY_SCREEN) && !assign_streams(c.Gk, c.rK) &&
           (c.rK == 16 || c.rK == 32);
}

void derive(sparsepr_ctx& c) {
    const sparsepr_params& p = c.p;
    c.H = p.heads;
    c.N = p.n;
    c.d = p.d;
    c.Gk = p.kv_groups;
    c.Gq = p.q_groups;
    c.rK = p.key_rank;
    c.raw = (p.flags & SPARSEPR_F_RAW_KMEANS) != 0;
    c.svoo = (p.flags & SPARSEPR_F_SVOO) != 0;
    c.fp8 = (p.flags & SPARSEPR_F_FP8_QK) != 0;
    c.Dq = c.d;                         // the query metric is used in full (d x d)
    c.k = routed_count(p.density, c.Gk);
    c.P = p.probes;
    c.T = p.kmeans_iters;
    c.nblk = (c.N + kSortChunk - 1) / kSortChunk;
    c.maxu = (c.N + kSparseRows - 1) / kSparseRows + c.Gq;
    // The fp8-logit experiment keeps 4-wave units only (its fp8 K tiles split over 256 lanes).
    // Below 2^17 query rows a call (512 units of 256 rows, two rounds of the CUs) the second
    // launch and its stream fork and join cost more than the longer walks save.
    c.big_units = !c.fp8 && !(p.flags & SPARSEPR_F_UNIFORM_UNITS) && (int64_t)c.H * c.N >= kBigUnitsMinRows;
    c.maxu_big = c.N / kDenseRows + c.Gq;     // whole 256-row chunks, one rest per group
    c.dense_units = (c.N + kDenseRows - 1) / kDenseRows;
    c.splits = probe_splits(c.N, c.H, c.P);
    c.gmax = std::max(c.Gk, c.Gq);
    c.weyl_a = weyl_multiplier(c.N);
    c.dev_eig = !c.raw && !c.svoo && !(p.flags & SPARSEPR_F_HOST_SOLVE) && c.rK <= kEigMaxR &&
                c.d <= kEigMaxN;
    c.nparts = (p.flags & SPARSEPR_F_SERIAL_PARTITION) ? 1 : std::min(c.H, kPartitionStreams);
}

void layout(sparsepr_ctx& c, Arena& a) {
    const size_t H = c.H, N = c.N, d = c.d, HN = H * N, HND = HN * d;
    const size_t P = std::max(c.P, 1);
    if (c.p.dtype == SPARSEPR_F32) {
        a.take(c.qb, HND);
        a.take(c.kb, HND);
        a.take(c.vb, HND);
    }
    a.take(c.kp, HND);
    a.take(c.vp, HND);
    a.take(c.vmax, H);
    if (c.fp8) {
        a.take(c.kp8, HND);
        a.take(c.qmax, H);
        a.take(c.kmax, H);
    }
    a.take(c.nonfinite, 2);
    a.take(c.klab, HN);
    a.take(c.qlab, HN);
    a.take(c.kperm, HN);
    a.take(c.qperm, HN);
    a.take(c.koff, H * (c.Gk + 1));
    a.take(c.qoff, H * (c.Gq + 1));
    a.take(c.flag_cnt, 2 * (size_t)c.T * H);
    a.take(c.flag_list, HN);
    if (assign_streams(c.Gq, (int)d) || assign_streams(c.Gk, (int)d)) {
        a.take(c.cand, HN * kMaxCandidates);
        a.take(c.ncand, HN);
        a.take(c.crow, H * c.gmax * d);
        a.take(c.ovf_cnt, H);
        a.take(c.ovf_list, HN);
        if (assign_streams(c.Gk, (int)d) && !c.raw && !c.svoo && c.rK <= kCandidateMaxDim)
            a.take(c.ycoord, HN * c.rK);
    }
    if (key_screen_in_coords(c)) {
        a.take(c.zhl, HN * 2 * c.rK);
        a.take(c.zkb, HN);
    }
    a.take(c.blkhist, H * c.nblk * c.gmax);
    a.take(c.blkoff, H * c.nblk * c.gmax);
    a.take(c.mk, H * d * d);
    a.take(c.w64, H * d * c.rK);
    if (c.dev_eig) {
        a.take(c.eig_diag, H * d);
        a.take(c.eig_off, H * d);
        a.take(c.eig_hv, H * d * d);
        a.take(c.eig_beta, H * d);
        a.take(c.eig_lam, H * (c.rK + 1));
        a.take(c.eig_vec, H * c.rK * d);
        a.take(c.eig_tnorm, H);
    }
    a.take(c.mgap, H);
    a.take(c.kc64, H * c.Gk * (c.raw || c.svoo ? d : (size_t)c.rK));
    if (c.raw) a.take(c.ident, H * d * d);
    a.take(c.qc64, H * c.Gq * d);
    a.take(c.kc2, H * c.Gk);
    a.take(c.qc2, H * c.Gq);
    a.take(c.kraw, H * c.Gk * d);
    a.take(c.kraw_t, H * c.Gk * d);
    a.take(c.qraw, H * c.Gq * d);
    a.take(c.kcp, H * 2 * c.Gk * d);
    a.take(c.qcp, H * 2 * c.Gq * d);
    a.take(c.kcn2, H * c.Gk);
    a.take(c.qcn2, H * c.Gq);
    a.take(c.kcpn, H * c.Gk);
    a.take(c.qcpn, H * c.Gq);
    a.take(c.blocks, H * c.Gq * c.k);
    a.take(c.ucount, H * c.Gq);
    a.take(c.probe_pos, H * P);
    a.take(c.probe_orig, H * P);
    a.take(c.probe_grp, H * P);
    a.take(c.probe_of, HN);
    a.take(c.nunits, H);
    a.take(c.units, H * c.maxu);
    a.take(c.nunits_big, H);
    a.take(c.units_big, H * c.maxu_big);
    a.take(c.pairs, H);
    a.take(c.o_s, HND);
    a.take(c.part_ml, H * c.splits * P * 4);
    a.take(c.part_od, H * c.splits * P * d);
    a.take(c.part_os, H * c.splits * P * d);
    a.take(c.px, H * P * d);
    a.take(c.py, H * P * d);
    a.take(c.pod, H * P * d);
    a.take(c.fit_m, H * 2 * d);
    a.take(c.fit_g, H * 3 * d * d);
    a.take(c.mq, H * d * d);
    a.take(c.bt16, H * 2 * d * d);
    a.take(c.bv32, H * d);
    a.take(c.dense_meta, 8);
    a.take(c.dense_unit_list, c.dense_units);
}

// fn(h) for every head on the context's host workers (up to 16 threads with the caller)
void parallel_heads(sparsepr_ctx* c, int heads, const std::function<void(int)>& fn) {
    const int hw = std::max(1u, std::thread::hardware_concurrency());
    const int nt = std::min(hw, 16);
    if (nt <= 1 || heads <= 1) {
        for (int h = 0; h < heads; ++h) fn(h);
        return;
    }
    if (!c->pool) c->pool.reset(new HostPool(nt - 1));
    c->pool->run(heads, fn);
}

int32_t fail(sparsepr_ctx* c, int32_t code, const std::string& msg) {
    if (c) {
        c->err = msg;
        if (code == SPARSEPR_ERR_HIP) c->poisoned = true;
    }
    return code;
}

#define SPR_HIP(ctx, expr)                                                                  \
    do {                                                                                    \
        hipError_t e_ = (expr);                                                             \
        if (e_ != hipSuccess)                                                               \
            return fail((ctx), SPARSEPR_ERR_HIP, std::string(#expr ": ") + hipGetErrorString(e_)); \
    } while (0)

#define SPR_LAUNCHED(ctx, what)                                                             \
    do {                                                                                    \
        hipError_t e_ = hipGetLastError();                                                  \
        if (e_ != hipSuccess)                                                               \
            return fail((ctx), SPARSEPR_ERR_HIP, std::string(what ": ") + hipGetErrorString(e_)); \
    } while (0)

int32_t enter(sparsepr_ctx* c, int need_stage) {
    if (!c) return SPARSEPR_ERR_INVALID_ARG;
    if (c->poisoned) return fail(c, SPARSEPR_ERR_HIP, "context poisoned by an earlier HIP error");
    if (c->stage < need_stage) return fail(c, SPARSEPR_ERR_ORDER, "stage called before its prerequisite");
    if (hipSetDevice(c->device) != hipSuccess) return fail(c, SPARSEPR_ERR_HIP, "hipSetDevice");
    return SPARSEPR_OK;
}

void mark(sparsepr_ctx* c, int point, hipStream_t st) {
    if (c->timing && hipEventRecord(c->ev[c->slot][point], st) == hipSuccess)
        c->ev_used[c->slot][point] = true;
}

// A new call starts at the partition stage: take the next ring slot.
void begin_call(sparsepr_ctx* c) {
    c->slot = static_cast<int>(c->calls % sparsepr_ctx::kRing);
    ++c->calls;
    for (bool& u : c->ev_used[c->slot]) u = false;
}

// bf16 view of an input tensor (converted into the workspace when the dtype is fp32)
const bf16_t* as_bf16(sparsepr_ctx* c, const void* x, bf16_t* scratch, hipStream_t st) {
    if (c->p.dtype == SPARSEPR_BF16) return static_cast<const bf16_t*>(x);
    launch_to_bf16(static_cast<const float*>(x), scratch, (size_t)c->H * c->N * c->d, st);
    return scratch;
}

bool aligned16(const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; }

// Lloyd rounds on the device: assign (MFMA screening, certified) -> fp64 recheck ->
// counting sort -> fp64 means and centroids. The metric is the factor l64 [d][dim], or
// with dim == 0 the full metric l64 [d][d]. After the last round `sorted`/`off` are the
// stable group-major permutation and `mean_raw` the raw group means (zero if empty).
// The fp64 recheck of the queued points of heads h0 .. h0 + hh - 1 (x, l64, c64, c2_64,
// labels, flags already offset to h0): with streamed centroids (large G) the queue is
// screened again for candidate lists first, so that only those are checked.
int32_t recheck(sparsepr_ctx* c, int h0, int hh, const bf16_t* x, int dim, const double* l64,
                const double* c64, const double* c2_64, const bf16_t* cpart, const float* cn2,
                const float* cpn, int groups, const int32_t* fc, int32_t* labels, hipStream_t st,
                const bf16_t* zhl = nullptr, const float* zkb = nullptr) {
    const size_t h = h0, N = c->N;
    const int32_t* flag_list = c->flag_list + h * N;
    if (c->cand && assign_streams(groups, c->d) && dim <= kCandidateMaxDim) {
        int32_t* cand = c->cand + h * N * kMaxCandidates;
        int32_t* ncand = c->ncand + h * N;
        int32_t* ovf_cnt = c->ovf_cnt + h;
        int32_t* ovf_list = c->ovf_list + h * N;
        // with zhl the keys were screened in their split coordinates: their candidates too
        launch_candidates(x, hh, c->N, c->d, cpart, cn2, cpn, groups, fc, flag_list, cand, ncand, ovf_cnt,
                          ovf_list, st, zhl, zkb, dim);
        const double* yc = (dim > 0 && c->ycoord) ? c->ycoord + h * N * dim : nullptr;
        launch_recheck_cand(x, hh, c->N, c->d, l64, dim, c->crow + h * c->gmax * c->d, c2_64, groups, fc,
                            flag_list, cand, ncand, yc, labels, st);
        launch_recheck(x, hh, c->N, c->d, l64, dim, c64, c2_64, groups, ovf_cnt, ovf_list, labels, st);
    } else {
        launch_recheck(x, hh, c->N, c->d, l64, dim, c64, c2_64, groups, fc, flag_list, labels, st);
    }
    SPR_LAUNCHED(c, "recheck");
    return SPARSEPR_OK;
}

// round: -1 enqueues the seeds only, 0 .. T-1 that Lloyd round only, kAllRounds the seeds
// and every round (the partition interleaves the rounds of its head groups' streams so that
// every stream is fed as the host enqueues).
constexpr int kAllRounds = -2;
int32_t lloyd(sparsepr_ctx* c, int h0, int hh, const bf16_t* x, int dim, const double* l64, int groups,
              int32_t* labels, int32_t* flags, int32_t* sorted, int32_t* off, double* mean_raw,
              double* c64, bf16_t* cpart, float* cn2, float* cpn, double* c2_64, hipStream_t st,
              const bf16_t* zhl = nullptr, const float* zkb = nullptr, int round = kAllRounds) {
    // heads h0 .. h0 + hh - 1: every buffer is head-major, so the slice starts h0 heads in
    const size_t h = h0, N = c->N, d = c->d, cdim = dim > 0 ? dim : c->d;
    x += h * N * d;
    l64 += h * d * cdim;
    labels += h * N;
    sorted += h * N;
    off += h * (groups + 1);
    mean_raw += h * groups * d;
    c64 += h * groups * cdim;
    cpart += h * 2 * groups * d;
    cn2 += h * groups;
    cpn += h * groups;
    c2_64 += h * groups;
    int32_t* flag_list = c->flag_list + h * N;
    // per-head-group bases at gmax strides: a group's key side and another's query side
    // (different G) run at once and must not share rows
    int32_t* blkhist = c->blkhist + h * c->nblk * c->gmax;
    int32_t* blkoff = c->blkoff + h * c->nblk * c->gmax;
    // each head group's rows start at h0 gmax d: the key side's narrower rows and the query
    // side's wider ones of two groups running at once never overlap
    double* crow = c->crow ? c->crow + h * c->gmax * c->d : nullptr;
    // zhl, zkb (the factor side only): screen in the coordinates x W, split, instead of x
    const int coords = zhl != nullptr;
    if (coords) {
        zhl += h * N * 2 * dim;
        zkb += h * N;
    }
    if (round == kAllRounds || round == -1) {
        launch_seed_centroids(x, hh, c->N, c->d, l64, dim, groups, c->weyl_a, mean_raw, c64, cpart, cn2,
                              cpn, c2_64, st, crow, coords);
        SPR_LAUNCHED(c, "seed centroids");
    }
    const int t0 = round == kAllRounds ? 0 : std::max(round, 0);
    const int t1 = round == kAllRounds ? c->T : (round < 0 ? 0 : round + 1);
    for (int t = t0; t < t1; ++t) {
        int32_t* fc = flags + (size_t)t * c->H + h;
        launch_assign(x, hh, c->N, c->d, cpart, cn2, cpn, groups, labels, fc, flag_list, st, zhl, zkb, dim);
        SPR_LAUNCHED(c, "assign");
        int32_t rc = recheck(c, h0, hh, x, dim, l64, c64, c2_64, cpart, cn2, cpn, groups, fc, labels, st,
                             zhl, zkb);
        if (rc) return rc;
        launch_counting_sort(labels, hh, c->N, groups, blkhist, blkoff, sorted, off, st);
        SPR_LAUNCHED(c, "counting sort");
        // the last round's raw means are the result; the screening vectors, metric-space
        // centroids and row copies that the finish derives from them would feed only a
        // further round, so it is skipped there
        launch_group_means(x, hh, c->N, c->d, sorted, off, groups, mean_raw, t + 1 < c->T ? l64 : nullptr,
                           dim, c64, cpart, cn2, cpn, c2_64, st, crow, coords);
        SPR_LAUNCHED(c, "group means");
    }
    return SPARSEPR_OK;
}

}  // namespace

namespace {
// why this thread's last sparsepr_create or context-free call failed
thread_local std::string create_err;
}  // namespace

namespace spr {
void set_call_error(const char* msg) { create_err = msg; }
}  // namespace spr

extern "C" {

int32_t sparsepr_validate(const sparsepr_params* p) { return validate(p); }

int32_t sparsepr_routed_count(const sparsepr_params* p) {
    const int32_t v = validate(p);
    return v != SPARSEPR_OK ? -v : routed_count(p->density, p->kv_groups);
}

size_t sparsepr_workspace_bytes(const sparsepr_params* p) {
    if (validate(p) != SPARSEPR_OK) return 0;
    sparsepr_ctx c;
    c.p = *p;
    derive(c);
    Arena a;
    layout(c, a);
    return a.used;
}

const char* sparsepr_status_str(int32_t s) {
    switch (s) {
        case SPARSEPR_OK: return "ok";
        case SPARSEPR_ERR_INVALID_ARG: return "invalid argument";
        case SPARSEPR_ERR_SHAPE: return "unsupported shape";
        case SPARSEPR_ERR_OOM: return "out of memory";
        case SPARSEPR_ERR_HIP: return "HIP error";
        case SPARSEPR_ERR_ORDER: return "stage order";
        case SPARSEPR_ERR_NUMERIC: return "numerical failure";
        default: return "unknown status";
    }
}

namespace {
int32_t create_fail(sparsepr_ctx* c, int32_t status, const char* what, hipError_t e) {
    create_err = std::string(what) + ": " + hipGetErrorString(e);
    if (c) sparsepr_destroy(c);
    return status;
}
}  // namespace

const char* sparsepr_last_error(const sparsepr_ctx* c) { return c ? c->err.c_str() : create_err.c_str(); }

int32_t sparsepr_create(const sparsepr_params* p, sparsepr_ctx** out) {
    if (!out) return SPARSEPR_ERR_INVALID_ARG;
    const int32_t v = validate(p);
    if (v != SPARSEPR_OK) return v;
    sparsepr_ctx* c = new (std::nothrow) sparsepr_ctx();
    if (!c) return SPARSEPR_ERR_OOM;
    c->p = *p;
    derive(*c);
    c->timing = (p->flags & SPARSEPR_F_STAGE_TIMING) != 0;
    c->check_finite = (p->flags & SPARSEPR_F_CHECK_FINITE) != 0;
    c->h_mgap.assign(p->heads, 0.0);
    c->h_rgap.assign(p->heads, INFINITY);
    hipError_t e;
    if ((e = hipGetDevice(&c->device)) != hipSuccess) {
        delete c;
        return create_fail(nullptr, SPARSEPR_ERR_HIP, "hipGetDevice", e);
    }
    Arena a;
    layout(*c, a);
    c->arena_bytes = a.used;
    if ((e = hipMalloc(&c->arena, c->arena_bytes)) != hipSuccess) {
        delete c;
        return create_fail(nullptr, SPARSEPR_ERR_OOM, "hipMalloc (arena)", e);
    }
    Arena b;
    b.base = static_cast<char*>(c->arena);
    layout(*c, b);
    if (c->timing)
        for (auto& row : c->ev)
            for (auto& ev : row)
                if (hipEventCreate(&ev) != hipSuccess) ev = nullptr;
    {
        const size_t H = c->H, d = c->d;
        if ((e = hipHostMalloc(reinterpret_cast<void**>(&c->h_fit), sizeof(double) * H * (2 * d + 3 * d * d))) != hipSuccess ||
            (e = hipHostMalloc(reinterpret_cast<void**>(&c->h_mkp), sizeof(double) * H * d * d)) != hipSuccess ||
            (e = hipHostMalloc(reinterpret_cast<void**>(&c->h_wp), sizeof(double) * H * d * c->rK)) != hipSuccess ||
            (e = hipHostMalloc(&c->h_b32, sizeof(float) * H * (d * d + d))) != hipSuccess)
            return create_fail(c, SPARSEPR_ERR_OOM, "hipHostMalloc", e);
        if ((e = hipEventCreateWithFlags(&c->ev_probe, hipEventDisableTiming)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&c->ev_rows, hipEventDisableTiming)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&c->ev_kdone, hipEventDisableTiming)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&c->ev_kperm, hipEventDisableTiming)) != hipSuccess ||
            (e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking)) != hipSuccess)
            return create_fail(c, SPARSEPR_ERR_HIP, "event / side stream", e);
        if (c->big_units &&
            ((e = hipEventCreateWithFlags(&c->ev_ufork, hipEventDisableTiming)) != hipSuccess ||
             (e = hipEventCreateWithFlags(&c->ev_ujoin, hipEventDisableTiming)) != hipSuccess ||
             (e = hipStreamCreateWithFlags(&c->ustream, hipStreamNonBlocking)) != hipSuccess))
            return create_fail(c, SPARSEPR_ERR_HIP, "event / work-unit stream", e);
        if (c->fp8 && (e = hipEventCreateWithFlags(&c->ev_qside, hipEventDisableTiming)) != hipSuccess)
            return create_fail(c, SPARSEPR_ERR_HIP, "event (fp8 scales)", e);
        if (c->nparts > 1 && (e = hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming)) != hipSuccess)
            return create_fail(c, SPARSEPR_ERR_HIP, "event (partition fork)", e);
        for (int i = 1; i < c->nparts; ++i)
            if ((e = hipEventCreateWithFlags(&c->ev_kd[i], hipEventDisableTiming)) != hipSuccess ||
                (e = hipEventCreateWithFlags(&c->ev_jn[i], hipEventDisableTiming)) != hipSuccess ||
                (e = hipStreamCreateWithFlags(&c->pstream[i], hipStreamNonBlocking)) != hipSuccess)
                return create_fail(c, SPARSEPR_ERR_HIP, "event / partition stream", e);
    }
    if (c->raw) {
        const size_t H = c->H, d = c->d;
        std::vector<double> eye(H * d * d, 0.0);
        for (size_t h = 0; h < H; ++h)
            for (size_t i = 0; i < d; ++i) eye[(h * d + i) * d + i] = 1.0;
        if ((e = hipMemcpy(c->ident, eye.data(), sizeof(double) * H * d * d, hipMemcpyHostToDevice)) != hipSuccess)
            return create_fail(c, SPARSEPR_ERR_HIP, "hipMemcpy (identity metric)", e);
    }
    // dense baseline metadata
    const int meta[8] = {0, c->N, 0, c->N, 0, c->dense_units, 0, 0};
    if ((e = hipMemcpy(c->dense_meta, meta, sizeof(meta), hipMemcpyHostToDevice)) != hipSuccess)
        return create_fail(c, SPARSEPR_ERR_HIP, "hipMemcpy (metadata)", e);
    launch_units(c->dense_meta, 1, 1, kDenseRows, c->dense_units, c->dense_unit_list,
                 c->dense_meta + 6, nullptr);
    if ((e = hipGetLastError()) != hipSuccess)
        return create_fail(c, SPARSEPR_ERR_HIP, "launch (dense work units)", e);
    if ((e = hipDeviceSynchronize()) != hipSuccess)
        return create_fail(c, SPARSEPR_ERR_HIP, "hipDeviceSynchronize (create)", e);
    create_err.clear();
    *out = c;
    return SPARSEPR_OK;
}

void sparsepr_destroy(sparsepr_ctx* c) {
    if (!c) return;
    (void)hipSetDevice(c->device);
    (void)hipDeviceSynchronize();
    if (c->timing)
        for (auto& row : c->ev)
            for (auto& e : row)
                if (e) (void)hipEventDestroy(e);
    if (c->ev_probe) (void)hipEventDestroy(c->ev_probe);
    if (c->ev_rows) (void)hipEventDestroy(c->ev_rows);
    if (c->ev_kdone) (void)hipEventDestroy(c->ev_kdone);
    if (c->ev_kperm) (void)hipEventDestroy(c->ev_kperm);
    if (c->ev_qside) (void)hipEventDestroy(c->ev_qside);
    if (c->side) (void)hipStreamDestroy(c->side);
    if (c->ustream) (void)hipStreamDestroy(c->ustream);
    if (c->ev_ufork) (void)hipEventDestroy(c->ev_ufork);
    if (c->ev_ujoin) (void)hipEventDestroy(c->ev_ujoin);
    if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
    for (int i = 1; i < sparsepr_ctx::kMaxParts; ++i) {
        if (c->ev_kd[i]) (void)hipEventDestroy(c->ev_kd[i]);
        if (c->ev_jn[i]) (void)hipEventDestroy(c->ev_jn[i]);
        if (c->pstream[i]) (void)hipStreamDestroy(c->pstream[i]);
    }
    if (c->h_fit) (void)hipHostFree(c->h_fit);
    if (c->h_mkp) (void)hipHostFree(c->h_mkp);
    if (c->h_wp) (void)hipHostFree(c->h_wp);
    if (c->h_b32) (void)hipHostFree(c->h_b32);
    if (c->arena) (void)hipFree(c->arena);
    delete c;
}

namespace {
// K into group-major order on the side stream, overlapping the query side of the
// partition; the sparse stage waits for ev_kperm before reading it. The side stream
// starts after all work enqueued so far on st, which includes the previous call's
// readers of the permuted K.
// SPARSEPR_F_FP8_QK: the per-head largest |q| and |k| on the side stream, after this
// stream's work so far (which includes the previous call's readers of them); the side
// stream's fp8 K permute and ev_kperm, which the sparse stage waits for, come after them.
int32_t fp8_scales_side(sparsepr_ctx* c, const bf16_t* q16, const bf16_t* k16, hipStream_t st) {
    if (!c->fp8) return SPARSEPR_OK;
    SPR_HIP(c, hipEventRecord(c->ev_qside, st));
    SPR_HIP(c, hipStreamWaitEvent(c->side, c->ev_qside, 0));
    launch_absmax_v(q16, c->H, c->N, c->d, c->qmax, c->side);
    launch_absmax_v(k16, c->H, c->N, c->d, c->kmax, c->side);
    SPR_LAUNCHED(c, "Q and K magnitudes (fp8)");
    return SPARSEPR_OK;
}

int32_t permute_keys_side(sparsepr_ctx* c, const bf16_t* k16, hipStream_t st) {
    SPR_HIP(c, hipEventRecord(c->ev_kdone, st));
    SPR_HIP(c, hipStreamWaitEvent(c->side, c->ev_kdone, 0));
    launch_permute(k16, c->kperm, c->H, c->N, c->d, c->kp, c->side);
    SPR_LAUNCHED(c, "permute K");
    if (c->fp8) {
        launch_permute_k8(k16, c->kperm, c->H, c->N, c->d, c->kmax, c->kp8, c->side);
        SPR_LAUNCHED(c, "permute K (fp8)");
    }
    SPR_HIP(c, hipEventRecord(c->ev_kperm, c->side));
    c->kperm_recorded = true;
    return SPARSEPR_OK;
}
}  // namespace

namespace {
// Comparison partitioner (SPARSEPR_F_SVOO): alternating rounds of one key assignment in the
// affinity space of the current query centroids (metric C_Q^T C_Q / d, in c->mk) and one
// query assignment in that of the updated key centroids (C_K^T C_K / d, in c->mq). Each
// assignment is one round of the method's Lloyd machinery in full-metric mode (certified
// MFMA screen, fp64 recheck, counting sort, fp64 raw means); the screening tables are rebuilt
// from the raw means under each new metric, empty groups included (zero centroid).
int32_t partition_svoo(sparsepr_ctx* c, const bf16_t* q16, const bf16_t* k16, hipStream_t st) {
    const int H = c->H, N = c->N, d = c->d;
    int32_t rc;
    launch_seed_raw(k16, H, N, d, c->Gk, c->weyl_a, c->kraw, st);
    launch_seed_raw(q16, H, N, d, c->Gq, c->weyl_a, c->qraw, st);
    SPR_LAUNCHED(c, "co-clustering seeds");
    for (int t = 0; t < c->T; ++t) {
        int32_t* fk = c->flag_cnt + (size_t)t * H;
        int32_t* fq = c->flag_cnt + (size_t)(c->T + t) * H;
        // keys against the current query centroids
        launch_gram_f64(c->qraw, H, c->Gq, d, 1.0 / d, c->mk, st);
        launch_finish_all(c->kraw, H, d, c->mk, 0, c->Gk, c->kc64, c->kcp, c->kcn2, c->kcpn, c->kc2, st, c->crow);
        launch_assign(k16, H, N, d, c->kcp, c->kcn2, c->kcpn, c->Gk, c->klab, fk, c->flag_list, st);
        if ((rc = recheck(c, 0, H, k16, 0, c->mk, c->kc64, c->kc2, c->kcp, c->kcn2, c->kcpn, c->Gk, fk,
                          c->klab, st)))
            return rc;
        launch_counting_sort(c->klab, H, N, c->Gk, c->blkhist, c->blkoff, c->kperm, c->koff, st);
        launch_group_means(k16, H, N, d, c->kperm, c->koff, c->Gk, c->kraw, nullptr, 0, nullptr, nullptr,
                           nullptr, nullptr, nullptr, st);
        SPR_LAUNCHED(c, "co-clustering keys");
        // queries against the updated key centroids
        launch_gram_f64(c->kraw, H, c->Gk, d, 1.0 / d, c->mq, st);
        launch_finish_all(c->qraw, H, d, c->mq, 0, c->Gq, c->qc64, c->qcp, c->qcn2, c->qcpn, c->qc2, st, c->crow);
        launch_assign(q16, H, N, d, c->qcp, c->qcn2, c->qcpn, c->Gq, c->qlab, fq, c->flag_list, st);
        if ((rc = recheck(c, 0, H, q16, 0, c->mq, c->qc64, c->qc2, c->qcp, c->qcn2, c->qcpn, c->Gq, fq,
                          c->qlab, st)))
            return rc;
        launch_counting_sort(c->qlab, H, N, c->Gq, c->blkhist, c->blkoff, c->qperm, c->qoff, st);
        launch_group_means(q16, H, N, d, c->qperm, c->qoff, c->Gq, c->qraw, nullptr, 0, nullptr, nullptr,
                           nullptr, nullptr, nullptr, st);
        SPR_LAUNCHED(c, "co-clustering queries");
    }
    return permute_keys_side(c, k16, st);
}

// Keys of heads h0 .. h0 + hh - 1 on stream s, one Lloyd step (round -1: the key
// coordinates and the seeds): Lloyd in the M_K eigen-coordinates W (already in c->w64);
// keys_done is recorded after the last round.
int32_t partition_keys(sparsepr_ctx* c, int h0, int hh, const bf16_t* k16, hipStream_t s,
                       hipEvent_t keys_done, int round) {
    const size_t h = h0, d = c->d;
    if (round == -1 && c->ycoord) {                    // every key's W coordinates, for the candidate recheck
        launch_coords(k16 + h * c->N * d, hh, c->N, c->d, c->w64 + h * d * c->rK, c->rK,
                      c->ycoord + h * c->N * c->rK, s);
        SPR_LAUNCHED(c, "key coordinates");
    }
    if (round == -1 && c->zhl) {        // the same coordinates, split, for the key screen
        launch_zcoords(k16 + h * c->N * d, hh, c->N, c->d, c->w64 + h * d * c->rK, c->rK,
                       c->zhl + h * c->N * 2 * c->rK, c->zkb + h * c->N, s);
        SPR_LAUNCHED(c, "key coordinates (screen)");
    }
    int32_t rc = lloyd(c, h0, hh, k16, c->rK, c->w64, c->Gk, c->klab, c->flag_cnt, c->kperm, c->koff,
                       c->kraw, c->kc64, c->kcp, c->kcn2, c->kcpn, c->kc2, s, c->zhl, c->zkb, round);
    if (rc) return rc;
    if (round == c->T - 1) SPR_HIP(c, hipEventRecord(keys_done, s));
    return SPARSEPR_OK;
}

// Queries of heads h0 .. h0 + hh - 1 on stream s, one Lloyd step (round -1: the
// logit-profile metric M = C_K^T C_K / d, the fp64 Gram of the raw key centroids used in
// full on the device, and the seeds).
int32_t partition_queries(sparsepr_ctx* c, int h0, int hh, const bf16_t* q16, hipStream_t s, int round) {
    const size_t h = h0, d = c->d;
    if (round == -1) {
        launch_gram_f64(c->kraw + h * c->Gk * d, hh, c->Gk, c->d, 1.0 / c->d, c->mq + h * d * d, s);
        SPR_LAUNCHED(c, "query metric");
    }
    return lloyd(c, h0, hh, q16, 0, c->mq, c->Gq, c->qlab, c->flag_cnt + (size_t)c->T * c->H, c->qperm,
                 c->qoff, c->qraw, c->qc64, c->qcp, c->qcn2, c->qcpn, c->qc2, s, nullptr, nullptr, round);
}

// Heads h0 .. h0 + hh - 1 of K (and of the V handed to sparsepr_attention) into group-major
// order on the side stream, once their keys are partitioned.
int32_t permute_group_side(sparsepr_ctx* c, int h0, int hh, const bf16_t* k16, hipEvent_t keys_done) {
    const size_t h = h0, nd = (size_t)c->N * c->d;
    SPR_HIP(c, hipStreamWaitEvent(c->side, keys_done, 0));
    launch_permute(k16 + h * nd, c->kperm + h * c->N, hh, c->N, c->d, c->kp + h * nd, c->side);
    SPR_LAUNCHED(c, "permute K");
    if (c->fp8) {
        launch_permute_k8(k16 + h * nd, c->kperm + h * c->N, hh, c->N, c->d, c->kmax + h, c->kp8 + h * nd,
                          c->side);
        SPR_LAUNCHED(c, "permute K (fp8)");
    }
    if (c->v_pre) {              // its magnitudes were taken during the eigensolve
        launch_permute_f16(c->v_pre + h * nd, c->kperm + h * c->N, hh, c->N, c->d, c->vmax + h,
                           c->vp + h * nd, c->side);
        SPR_LAUNCHED(c, "permute V");
    }
    return SPARSEPR_OK;
}

// The per-head steps run as nparts groups of consecutive heads, each on its own stream
// (group 0 on st), so that the many small, latency-bound launches of one group (recheck,
// sort, centroid finish) overlap the other groups' work; with SPARSEPR_F_SERIAL_PARTITION
// (or one head) all heads run on st. The other streams start after an event on st and are
// joined back into it. The host enqueues the groups' steps round by round, every group's keys
// before any group's queries, so that each stream is fed while the host works; each group's
// K (and V) is permuted on the side stream as soon as its keys are partitioned, overlapping
// the query side.
int32_t partition_keys_and_queries(sparsepr_ctx* c, const bf16_t* q16, const bf16_t* k16, hipStream_t st) {
    int32_t rc;
    const int np = c->nparts;
    if (np > 1) {
        SPR_HIP(c, hipEventRecord(c->ev_fork, st));
        for (int i = 1; i < np; ++i) SPR_HIP(c, hipStreamWaitEvent(c->pstream[i], c->ev_fork, 0));
    }
    auto group = [&](int i, int& h0, int& hh, hipStream_t& s, hipEvent_t& kd) {
        h0 = (int)((int64_t)c->H * i / np);
        hh = (int)((int64_t)c->H * (i + 1) / np) - h0;
        s = i == 0 ? st : c->pstream[i];
        kd = i == 0 ? c->ev_kdone : c->ev_kd[i];
    };
    int h0, hh;
    hipStream_t s;
    hipEvent_t kd;
    for (int r = -1; r < c->T; ++r)
        for (int i = 0; i < np; ++i) {
            group(i, h0, hh, s, kd);
            if ((rc = partition_keys(c, h0, hh, k16, s, kd, r))) return rc;
        }
    for (int i = 0; i < np; ++i) {
        group(i, h0, hh, s, kd);
        if ((rc = permute_group_side(c, h0, hh, k16, kd))) return rc;
    }
    if (c->v_pre) c->v_pre_done = true;
    SPR_HIP(c, hipEventRecord(c->ev_kperm, c->side));           // the sparse stage waits for it
    c->kperm_recorded = true;
    for (int r = -1; r < c->T; ++r)
        for (int i = 0; i < np; ++i) {
            group(i, h0, hh, s, kd);
            if ((rc = partition_queries(c, h0, hh, q16, s, r))) return rc;
        }
    for (int i = 1; i < np; ++i) {
        SPR_HIP(c, hipEventRecord(c->ev_jn[i], c->pstream[i]));
        SPR_HIP(c, hipStreamWaitEvent(st, c->ev_jn[i], 0));
    }
    mark(c, 1, st);
    c->stage = kStagePartition;
    return SPARSEPR_OK;
}
}  // namespace

int32_t sparsepr_partition(sparsepr_ctx* c, const void* q, const void* k, void* stream) {
    int32_t rc = enter(c, 0);
    if (rc) return rc;
    if (!q || !k || !aligned16(q) || !aligned16(k)) return fail(c, SPARSEPR_ERR_INVALID_ARG, "null or misaligned q/k");
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    c->stage = 0;
    begin_call(c);
    mark(c, 0, st);
    const size_t H = c->H, d = c->d, rK = c->rK;
    const bf16_t* q16 = as_bf16(c, q, c->qb, st);
    const bf16_t* k16 = as_bf16(c, k, c->kb, st);
    launch_fill_i32(c->flag_cnt, 0, 2 * (size_t)c->T * H, st);
    if (c->check_finite) {
        launch_fill_i64(reinterpret_cast<int64_t*>(c->nonfinite), 0, 2, st);
        launch_count_nonfinite(q16, H * c->N * d, 0, c->nonfinite, st);
        launch_count_nonfinite(k16, H * c->N * d, 0, c->nonfinite, st);
        SPR_LAUNCHED(c, "finite check (q, k)");
    }
    if ((rc = fp8_scales_side(c, q16, k16, st))) return rc;
    if (c->svoo) {
        std::fill(c->h_mgap.begin(), c->h_mgap.end(), 0.0);      // no M_K
        c->mgap_dev = false;
        if ((rc = partition_svoo(c, q16, k16, st))) return rc;
        mark(c, 1, st);
        c->stage = kStagePartition;
        return SPARSEPR_OK;
    }
    if (c->raw) {
        std::fill(c->h_mgap.begin(), c->h_mgap.end(), 0.0);      // no M_K
        c->mgap_dev = false;
        // comparison partitioner: plain Euclidean k-means of the raw key rows, then of the
        // raw query rows (full-metric path with M = I: screening vector = mean)
        rc = lloyd(c, 0, c->H, k16, 0, c->ident, c->Gk, c->klab, c->flag_cnt, c->kperm, c->koff, c->kraw,
                   c->kc64, c->kcp, c->kcn2, c->kcpn, c->kc2, st);
        if (rc) return rc;
        if ((rc = permute_keys_side(c, k16, st))) return rc;
        rc = lloyd(c, 0, c->H, q16, 0, c->ident, c->Gq, c->qlab, c->flag_cnt + (size_t)c->T * H, c->qperm,
                   c->qoff, c->qraw, c->qc64, c->qcp, c->qcn2, c->qcpn, c->qc2, st);
        if (rc) return rc;
        mark(c, 1, st);
        c->stage = kStagePartition;
        return SPARSEPR_OK;
    }
    if (c->v_pre) {
        // V (handed over by sparsepr_attention) needs the key permutation only for its
        // permute: its per-head magnitudes run on the side stream beside the metric and its
        // eigensolve, after the previous call's readers on this stream
        SPR_HIP(c, hipEventRecord(c->ev_kdone, st));
        SPR_HIP(c, hipStreamWaitEvent(c->side, c->ev_kdone, 0));
        launch_absmax_v(c->v_pre, c->H, c->N, c->d, c->vmax, c->side);
        SPR_LAUNCHED(c, "V magnitudes");
    }
    // M_K and its leading eigenvectors (fp64; on the device unless SPARSEPR_F_HOST_SOLVE)
    launch_metric(q16, c->H, c->N, c->d, c->p.n_sample, c->weyl_a, c->mk, st);
    SPR_LAUNCHED(c, "metric");
    c->mgap_dev = c->dev_eig;
    if (c->dev_eig) {
        launch_sym_eig_top(c->mk, c->H, c->d, c->rK, c->eig_diag, c->eig_off, c->eig_hv, c->eig_beta,
                           c->eig_lam, c->eig_vec, c->eig_tnorm, c->w64, c->mgap, st);
        SPR_LAUNCHED(c, "metric eigensolve");
        return partition_keys_and_queries(c, q16, k16, st);
    }
    // (pinned staging both ways; W is rewritten only after the next call's sync)
    SPR_HIP(c, hipMemcpyAsync(c->h_mkp, c->mk, sizeof(double) * H * d * d, hipMemcpyDeviceToHost, st));
    SPR_HIP(c, hipStreamSynchronize(st));
    std::vector<int> prc(H, 0);
    parallel_heads(c, (int)H, [&](int h) {
        std::fill(c->h_wp + h * d * rK, c->h_wp + (h + 1) * d * rK, 0.0);
        prc[h] = key_projection((int)d, c->h_mkp + h * d * d, (int)rK, c->h_wp + h * d * rK, &c->h_mgap[h]);
    });
    for (size_t h = 0; h < H; ++h) {
        if (prc[h] != 0) return fail(c, SPARSEPR_ERR_NUMERIC, "metric eigensolve failed (non-finite input)");
    }
    SPR_HIP(c, hipMemcpyAsync(c->w64, c->h_wp, sizeof(double) * H * d * rK, hipMemcpyHostToDevice, st));
    return partition_keys_and_queries(c, q16, k16, st);
}

int32_t sparsepr_set_partition(sparsepr_ctx* c, const void* q, const void* k,
                               const int32_t* key_labels, const int32_t* q_labels, int32_t host,
                               void* stream) {
    int32_t rc = enter(c, 0);
    if (rc) return rc;
    if (!q || !k || !key_labels || !q_labels || !aligned16(q) || !aligned16(k))
        return fail(c, SPARSEPR_ERR_INVALID_ARG, "null or misaligned argument");
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    const size_t HN = (size_t)c->H * c->N;
    if (host) {
        for (size_t i = 0; i < HN; ++i)
            if (key_labels[i] < 0 || key_labels[i] >= c->Gk || q_labels[i] < 0 || q_labels[i] >= c->Gq)
                return fail(c, SPARSEPR_ERR_INVALID_ARG, "label out of range");
    }
    const hipMemcpyKind kind = host ? hipMemcpyHostToDevice : hipMemcpyDeviceToDevice;
    SPR_HIP(c, hipMemcpyAsync(c->klab, key_labels, sizeof(int32_t) * HN, kind, st));
    SPR_HIP(c, hipMemcpyAsync(c->qlab, q_labels, sizeof(int32_t) * HN, kind, st));
    const bf16_t* q16 = as_bf16(c, q, c->qb, st);
    const bf16_t* k16 = as_bf16(c, k, c->kb, st);
    launch_fill_i32(c->flag_cnt, 0, 2 * (size_t)c->T * c->H, st);
    if ((rc = fp8_scales_side(c, q16, k16, st))) return rc;
    launch_counting_sort(c->klab, c->H, c->N, c->Gk, c->blkhist, c->blkoff, c->kperm, c->koff, st);
    if ((rc = permute_keys_side(c, k16, st))) return rc;
    launch_group_means(k16, c->H, c->N, c->d, c->kperm, c->koff, c->Gk, c->kraw, nullptr, 0, nullptr,
                       nullptr, nullptr, nullptr, nullptr, st);
    launch_counting_sort(c->qlab, c->H, c->N, c->Gq, c->blkhist, c->blkoff, c->qperm, c->qoff, st);
    launch_group_means(q16, c->H, c->N, c->d, c->qperm, c->qoff, c->Gq, c->qraw, nullptr, 0, nullptr,
                       nullptr, nullptr, nullptr, nullptr, st);
    SPR_LAUNCHED(c, "set partition");
    if (host) SPR_HIP(c, hipStreamSynchronize(st));   // host labels must stay valid until copied
    c->stage = kStagePartition;
    return SPARSEPR_OK;
}

int32_t sparsepr_route(sparsepr_ctx* c, const void* q, const void* k, const void* v, void* stream) {
    int32_t rc = enter(c, kStagePartition);
    if (rc) return rc;
    if (!q || !k || !v || !aligned16(q) || !aligned16(k) || !aligned16(v))
        return fail(c, SPARSEPR_ERR_INVALID_ARG, "null or misaligned q/k/v");
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    mark(c, 2, st);
    // K was permuted in the partition stage (side stream); q is recorded, not copied
    const bf16_t* q16 = as_bf16(c, q, c->qb, st);
    const bf16_t* v16 = as_bf16(c, v, c->vb, st);
    c->q_src = q16;           // the sparse stage gathers query rows through the permutation
    c->v_src = v16;           // and the probe rows gather bf16 V rows through the key permutation
    if (c->check_finite) {
        launch_count_nonfinite(v16, (size_t)c->H * c->N * c->d, 0, c->nonfinite, st);
        SPR_LAUNCHED(c, "finite check (v)");
    }
    if (!(c->v_pre_done && c->v_pre == v16)) {
        launch_permute_v16(v16, c->kperm, c->H, c->N, c->d, c->vmax, c->vp, st);
        SPR_LAUNCHED(c, "permute");
    }
    c->v_pre = nullptr;
    c->v_pre_done = false;
    launch_fill_i64(c->pairs, 0, c->H, st);
    launch_route(c->qraw, c->kraw, c->kraw_t, c->qoff, c->koff, c->H, c->Gq, c->Gk, c->d, c->k,
                 c->blocks, c->ucount, c->pairs, st);
    SPR_LAUNCHED(c, "route");
    launch_fill_i32(c->probe_of, -1, (size_t)c->H * c->N, st);
    launch_probes(c->qoff, c->qperm, c->H, c->N, c->Gq, c->P, c->probe_pos, c->probe_orig,
                  c->probe_grp, c->probe_of, st);
    launch_units(c->qoff, c->H, c->Gq, kSparseRows, c->maxu, c->units, c->nunits, st,
                 c->big_units ? kDenseRows : 0, c->maxu_big, c->units_big, c->nunits_big);
    SPR_LAUNCHED(c, "probes/units");
    mark(c, 3, st);
    c->stage = kStageRoute;
    c->have_route = true;
    return SPARSEPR_OK;
}

int32_t sparsepr_reuse_route(sparsepr_ctx* c, const void* q, const void* k, const void* v, void* stream) {
    int32_t rc = enter(c, 0);
    if (rc) return rc;
    if (!c->have_route) return fail(c, SPARSEPR_ERR_ORDER, "no earlier partition and routing to reuse");
    if (!q || !k || !v || !aligned16(q) || !aligned16(k) || !aligned16(v))
        return fail(c, SPARSEPR_ERR_INVALID_ARG, "null or misaligned q/k/v");
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    begin_call(c);
    mark(c, 0, st);
    mark(c, 1, st);                                     // no partition in this call
    mark(c, 2, st);
    const size_t HND = (size_t)c->H * c->N * c->d;
    const bf16_t* q16 = as_bf16(c, q, c->qb, st);
    const bf16_t* k16 = as_bf16(c, k, c->kb, st);
    const bf16_t* v16 = as_bf16(c, v, c->vb, st);
    if (c->check_finite) {
        launch_fill_i64(reinterpret_cast<int64_t*>(c->nonfinite), 0, 2, st);
        launch_count_nonfinite(q16, HND, 0, c->nonfinite, st);
        launch_count_nonfinite(k16, HND, 0, c->nonfinite, st);
        launch_count_nonfinite(v16, HND, 0, c->nonfinite, st);
        SPR_LAUNCHED(c, "finite check (q, k, v)");
    }
    c->q_src = q16;
    c->v_src = v16;
    // the new K and V through the kept key permutation; blocks, probes and work units stay
    if ((rc = fp8_scales_side(c, q16, k16, st))) return rc;
    if ((rc = permute_keys_side(c, k16, st))) return rc;
    launch_permute_v16(v16, c->kperm, c->H, c->N, c->d, c->vmax, c->vp, st);
    SPR_LAUNCHED(c, "permute");
    mark(c, 3, st);
    c->stage = kStageRoute;
    return SPARSEPR_OK;
}

int32_t sparsepr_sparse_attn(sparsepr_ctx* c, void* stream) {
    int32_t rc = enter(c, kStageRoute);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    const size_t H = c->H, d = c->d;
    // Probe rows first. The fit's fp64 means and Grams, and their copy to pinned host
    // memory, run on the side stream while the main kernel runs on this one; the host
    // solve (sparsepr_probe_fit) waits for them only. This stream first waits for the
    // previous call's side work, which reads the probe buffers written here.
    SPR_HIP(c, hipStreamWaitEvent(st, c->ev_probe, 0));
    SPR_HIP(c, hipStreamWaitEvent(st, c->ev_kperm, 0));        // K permuted (side stream)
    if (c->P > 0) {
        launch_probe(c->q_src, c->kp, c->v_src, c->kperm, c->H, c->N, c->d, c->probe_orig, c->probe_grp, c->P,
                     c->koff, c->Gk + 1, c->Gk, c->blocks, c->Gq, c->k, c->splits, c->part_ml,
                     c->part_od, c->part_os, st);
        launch_probe_merge(c->H, c->P, c->d, c->splits, c->part_ml, c->part_od, c->part_os, c->px,
                           c->py, c->pod, st);
        SPR_LAUNCHED(c, "probe rows");
        SPR_HIP(c, hipEventRecord(c->ev_rows, st));
        hipStream_t sd = c->side;
        SPR_HIP(c, hipStreamWaitEvent(sd, c->ev_rows, 0));
        double* xm = c->fit_m;
        double* ym = c->fit_m + H * d;
        double* gxx = c->fit_g;
        double* gxy = c->fit_g + H * d * d;
        double* gyy = c->fit_g + 2 * H * d * d;
        launch_col_means_f32(c->px, c->H, c->P, c->d, xm, sd);
        launch_col_means_f32(c->py, c->H, c->P, c->d, ym, sd);
        launch_gram_f32(c->px, c->px, xm, xm, c->H, c->P, c->d, gxx, sd);
        launch_gram_f32(c->px, c->py, xm, ym, c->H, c->P, c->d, gxy, sd);
        launch_gram_f32(c->py, c->py, nullptr, nullptr, c->H, c->P, c->d, gyy, sd);
        SPR_LAUNCHED(c, "fit grams");
        SPR_HIP(c, hipMemcpyAsync(c->h_fit, c->fit_m, sizeof(double) * H * 2 * d, hipMemcpyDeviceToHost, sd));
        SPR_HIP(c, hipMemcpyAsync(c->h_fit + H * 2 * d, c->fit_g, sizeof(double) * H * 3 * d * d,
                                  hipMemcpyDeviceToHost, sd));
        SPR_HIP(c, hipEventRecord(c->ev_probe, sd));
    } else {
        SPR_HIP(c, hipEventRecord(c->ev_probe, st));
    }
    mark(c, 4, st);
    // 256-row units in 8-wave blocks (one key-union walk for up to 256 rows: each group's
    // whole 256-row chunks and a rest of more than 128 rows) on this stream, and the shorter
    // rests in 128-row units (4-wave blocks, two per CU) on a stream of their own beside
    // them: the two write disjoint rows of O_s, and the small units fill the CUs that the
    // large ones' last round leaves idle.
    hipStream_t su = st;
    if (c->big_units) {
        SPR_HIP(c, hipEventRecord(c->ev_ufork, st));
        SPR_HIP(c, hipStreamWaitEvent(c->ustream, c->ev_ufork, 0));
        su = c->ustream;
        launch_vbsa(c->q_src, c->qperm, c->kp, c->vp, c->vmax, c->H, c->N, c->d, c->qoff, c->Gq + 1, c->koff,
                    c->Gk + 1, c->blocks, c->Gq * c->k, c->k, c->units_big, c->maxu_big, c->nunits_big, 1,
                    c->maxu_big, kDenseRows, c->o_s, 0, st);
    }
    launch_vbsa(c->q_src, c->qperm, c->kp, c->vp, c->vmax, c->H, c->N, c->d, c->qoff, c->Gq + 1, c->koff, c->Gk + 1,
                c->blocks, c->Gq * c->k, c->k, c->units, c->maxu, c->nunits, 1, c->maxu, kSparseRows,
                c->o_s, 0, su, c->fp8 ? c->kp8 : nullptr, c->qmax, c->kmax);
    if (c->big_units) {
        SPR_HIP(c, hipEventRecord(c->ev_ujoin, su));
        SPR_HIP(c, hipStreamWaitEvent(st, c->ev_ujoin, 0));
    }
    SPR_LAUNCHED(c, "sparse attention");
    mark(c, 5, st);
    c->stage = kStageAttn;
    return SPARSEPR_OK;
}

int32_t sparsepr_probe_fit(sparsepr_ctx* c, void* stream) {
    int32_t rc = enter(c, kStageAttn);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    const size_t H = c->H, d = c->d, P = c->P;
    c->h_bm.assign(H * d * d, 0.0);
    c->h_bv.assign(H * d, 0.0);
    c->h_rgap.assign(H, INFINITY);
    // waits for the probe rows and Grams only: the main kernel keeps running
    SPR_HIP(c, hipEventSynchronize(c->ev_probe));
    if (P > 0) {
        const double* hm = c->h_fit;
        const double* hg = c->h_fit + H * 2 * d;
        std::vector<int> frc(H, 0);
        parallel_heads(c, (int)H, [&](int h) {
            frc[h] = probe_fit_from_grams((int)P, (int)d, &hm[h * d], &hm[(H + h) * d], &hg[h * d * d],
                                          &hg[(H + h) * d * d], &hg[(2 * H + h) * d * d],
                                          c->p.ridge_lambda, c->p.corr_rank, &c->h_bm[h * d * d],
                                          &c->h_bv[h * d], &c->h_rgap[h]);
        });
        for (size_t h = 0; h < H; ++h)
            if (frc[h] != 0) return fail(c, SPARSEPR_ERR_NUMERIC, "probe fit failed (non-finite probe outputs)");
    }
    // (the previous call's upload from this buffer finished before ev_probe fired)
    // B'^T split into bf16 hi + lo (nearest even), the correction kernel's MFMA operand
    bf16_t* hb = static_cast<bf16_t*>(c->h_b32);
    float* hv = reinterpret_cast<float*>(hb + H * 2 * d * d);
    for (size_t h = 0; h < H; ++h)
        for (size_t j = 0; j < d; ++j)
            for (size_t i = 0; i < d; ++i) {
                const double b = c->h_bm[(h * d + i) * d + j];
                const bf16_t bh = f32_to_bf16(static_cast<float>(b));
                hb[((h * 2 + 0) * d + j) * d + i] = bh;
                hb[((h * 2 + 1) * d + j) * d + i] = f32_to_bf16(static_cast<float>(b - (double)bf16_to_f32(bh)));
            }
    for (size_t i = 0; i < H * d; ++i) hv[i] = (float)c->h_bv[i];
    SPR_HIP(c, hipMemcpyAsync(c->bt16, hb, sizeof(bf16_t) * H * 2 * d * d, hipMemcpyHostToDevice, st));
    SPR_HIP(c, hipMemcpyAsync(c->bv32, hv, sizeof(float) * H * d, hipMemcpyHostToDevice, st));
    mark(c, 6, st);
    c->stage = kStageFit;
    return SPARSEPR_OK;
}

int32_t sparsepr_correct(sparsepr_ctx* c, void* o, void* stream) {
    int32_t rc = enter(c, kStageFit);
    if (rc) return rc;
    if (!o || !aligned16(o)) return fail(c, SPARSEPR_ERR_INVALID_ARG, "null or misaligned o");
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    launch_correct(c->o_s, c->bt16, c->bv32, c->pod, c->probe_orig, c->qperm, c->H, c->N, c->d, c->P, o,
                   c->p.dtype == SPARSEPR_F32 ? 1 : 0, st);
    SPR_LAUNCHED(c, "correct");
    if (c->check_finite) {
        launch_count_nonfinite(o, (size_t)c->H * c->N * c->d, c->p.dtype == SPARSEPR_F32 ? 1 : 0,
                               c->nonfinite + 1, st);
        SPR_LAUNCHED(c, "finite check (o)");
    }
    mark(c, 7, st);
    c->stage = kStageCorrect;
    return SPARSEPR_OK;
}

int32_t sparsepr_attention(sparsepr_ctx* c, const void* q, const void* k, const void* v, void* o,
                           void* stream) {
    // bf16 V needs no conversion, so the partition stage can permute it beside the query side
    if (c && c->p.dtype == SPARSEPR_BF16 && v && aligned16(v)) c->v_pre = static_cast<const bf16_t*>(v);
    int32_t rc = sparsepr_partition(c, q, k, stream);
    if (!rc) rc = sparsepr_route(c, q, k, v, stream);
    if (c) {
        c->v_pre = nullptr;
        c->v_pre_done = false;
    }
    if (!rc) rc = sparsepr_sparse_attn(c, stream);
    if (!rc) rc = sparsepr_probe_fit(c, stream);
    if (!rc) rc = sparsepr_correct(c, o, stream);
    return rc;
}

int32_t sparsepr_attention_reuse(sparsepr_ctx* c, const void* q, const void* k, const void* v, void* o,
                                 void* stream) {
    int32_t rc = sparsepr_reuse_route(c, q, k, v, stream);
    if (!rc) rc = sparsepr_sparse_attn(c, stream);
    if (!rc) rc = sparsepr_probe_fit(c, stream);
    if (!rc) rc = sparsepr_correct(c, o, stream);
    return rc;
}

int32_t sparsepr_dense_attn(sparsepr_ctx* c, const void* q, const void* k, const void* v, void* o,
                            void* stream) {
    int32_t rc = enter(c, 0);
    if (rc) return rc;
    if (!q || !k || !v || !o || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(c, SPARSEPR_ERR_INVALID_ARG, "null or misaligned argument");
    hipStream_t st = static_cast<hipStream_t>(stream);
    c->last_stream = st;
    // the side stream's K permute may still read the bf16 copy of k rewritten here
    if (c->kperm_recorded) SPR_HIP(c, hipStreamWaitEvent(st, c->ev_kperm, 0));
    const bf16_t* q16 = as_bf16(c, q, c->qb, st);
    const bf16_t* k16 = as_bf16(c, k, c->kb, st);
    const bf16_t* v16 = as_bf16(c, v, c->vb, st);
    launch_vbsa(q16, nullptr, k16, v16, nullptr, c->H, c->N, c->d, c->dense_meta, 0, c->dense_meta + 2, 0,
                c->dense_meta + 4, 0, 1, c->dense_unit_list, 0, c->dense_meta + 6, 0, c->dense_units,
                kDenseRows, o, c->p.dtype == SPARSEPR_F32 ? 0 : 1, st);
    SPR_LAUNCHED(c, "dense attention");
    return SPARSEPR_OK;
}

// ---------------------------------------------------------------- inspection ---
static int32_t copy_out(sparsepr_ctx* c, void* dst, const void* src, size_t bytes, int32_t host,
                        hipStream_t st) {
    if (!dst) return SPARSEPR_OK;
    SPR_HIP(c, hipMemcpyAsync(dst, src, bytes, host ? hipMemcpyDeviceToHost : hipMemcpyDeviceToDevice, st));
    return SPARSEPR_OK;
}

int32_t sparsepr_get_partition(sparsepr_ctx* c, int32_t* key_labels, int32_t* q_labels,
                               int32_t* key_perm, int32_t* q_perm, int32_t* key_off, int32_t* q_off,
                               int32_t host, void* stream) {
    int32_t rc = enter(c, kStagePartition);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t HN = (size_t)c->H * c->N;
    if ((rc = copy_out(c, key_labels, c->klab, 4 * HN, host, st))) return rc;
    if ((rc = copy_out(c, q_labels, c->qlab, 4 * HN, host, st))) return rc;
    if ((rc = copy_out(c, key_perm, c->kperm, 4 * HN, host, st))) return rc;
    if ((rc = copy_out(c, q_perm, c->qperm, 4 * HN, host, st))) return rc;
    if ((rc = copy_out(c, key_off, c->koff, 4 * (size_t)c->H * (c->Gk + 1), host, st))) return rc;
    if ((rc = copy_out(c, q_off, c->qoff, 4 * (size_t)c->H * (c->Gq + 1), host, st))) return rc;
    if (host) SPR_HIP(c, hipStreamSynchronize(st));
    return SPARSEPR_OK;
}

int32_t sparsepr_get_routing(sparsepr_ctx* c, int32_t* blocks, int32_t* probe_orig, int32_t* probe_pos,
                             int32_t host, void* stream) {
    int32_t rc = enter(c, kStageRoute);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = copy_out(c, blocks, c->blocks, 4 * (size_t)c->H * c->Gq * c->k, host, st))) return rc;
    if (c->P > 0) {
        if ((rc = copy_out(c, probe_orig, c->probe_orig, 4 * (size_t)c->H * c->P, host, st))) return rc;
        if ((rc = copy_out(c, probe_pos, c->probe_pos, 4 * (size_t)c->H * c->P, host, st))) return rc;
    }
    if (host) SPR_HIP(c, hipStreamSynchronize(st));
    return SPARSEPR_OK;
}

int32_t sparsepr_get_metric(sparsepr_ctx* c, double* m_k, double* w, int32_t host, void* stream) {
    int32_t rc = enter(c, kStagePartition);
    if (rc) return rc;
    if (c->raw || c->svoo)
        return fail(c, SPARSEPR_ERR_ORDER, "no key metric with SPARSEPR_F_RAW_KMEANS or SPARSEPR_F_SVOO");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = copy_out(c, m_k, c->mk, 8 * (size_t)c->H * c->d * c->d, host, st))) return rc;
    if ((rc = copy_out(c, w, c->w64, 8 * (size_t)c->H * c->d * c->rK, host, st))) return rc;
    if (host) SPR_HIP(c, hipStreamSynchronize(st));
    return SPARSEPR_OK;
}

int32_t sparsepr_get_centroids(sparsepr_ctx* c, double* key_centroids, double* q_centroids, int32_t host,
                               void* stream) {
    int32_t rc = enter(c, kStagePartition);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = copy_out(c, key_centroids, c->kraw, 8 * (size_t)c->H * c->Gk * c->d, host, st))) return rc;
    if ((rc = copy_out(c, q_centroids, c->qraw, 8 * (size_t)c->H * c->Gq * c->d, host, st))) return rc;
    if (host) SPR_HIP(c, hipStreamSynchronize(st));
    return SPARSEPR_OK;
}

int32_t sparsepr_get_sparse_out(sparsepr_ctx* c, float* o_sparse, int32_t host, void* stream) {
    int32_t rc = enter(c, kStageAttn);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = copy_out(c, o_sparse, c->o_s, 4 * (size_t)c->H * c->N * c->d, host, st))) return rc;
    if (host) SPR_HIP(c, hipStreamSynchronize(st));
    return SPARSEPR_OK;
}

int32_t sparsepr_get_probes(sparsepr_ctx* c, float* x, float* y, int32_t host, void* stream) {
    int32_t rc = enter(c, kStageAttn);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (c->P > 0) {
        if ((rc = copy_out(c, x, c->px, 4 * (size_t)c->H * c->P * c->d, host, st))) return rc;
        if ((rc = copy_out(c, y, c->py, 4 * (size_t)c->H * c->P * c->d, host, st))) return rc;
    }
    if (host) SPR_HIP(c, hipStreamSynchronize(st));
    return SPARSEPR_OK;
}

int32_t sparsepr_get_fit(sparsepr_ctx* c, double* b_mat, double* b_vec, int32_t host, void* stream) {
    int32_t rc = enter(c, kStageFit);
    if (rc) return rc;
    const size_t H = c->H, d = c->d;
    if (host) {
        if (b_mat) std::memcpy(b_mat, c->h_bm.data(), 8 * H * d * d);
        if (b_vec) std::memcpy(b_vec, c->h_bv.data(), 8 * H * d);
        return SPARSEPR_OK;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (b_mat) SPR_HIP(c, hipMemcpyAsync(b_mat, c->h_bm.data(), 8 * H * d * d, hipMemcpyHostToDevice, st));
    if (b_vec) SPR_HIP(c, hipMemcpyAsync(b_vec, c->h_bv.data(), 8 * H * d, hipMemcpyHostToDevice, st));
    SPR_HIP(c, hipStreamSynchronize(st));
    return SPARSEPR_OK;
}

int32_t sparsepr_get_gaps(sparsepr_ctx* c, double* metric_gap, double* resid_gap, int32_t host,
                          void* stream) {
    int32_t rc = enter(c, kStagePartition);
    if (rc) return rc;
    if (!host) return fail(c, SPARSEPR_ERR_INVALID_ARG, "sparsepr_get_gaps writes host memory only");
    SPR_HIP(c, hipStreamSynchronize(static_cast<hipStream_t>(stream)));
    if (c->mgap_dev) SPR_HIP(c, hipMemcpy(c->h_mgap.data(), c->mgap, 8 * (size_t)c->H, hipMemcpyDeviceToHost));
    if (metric_gap) std::copy(c->h_mgap.begin(), c->h_mgap.end(), metric_gap);
    if (resid_gap) {
        if (c->stage >= kStageFit) std::copy(c->h_rgap.begin(), c->h_rgap.end(), resid_gap);
        else std::fill(resid_gap, resid_gap + c->H, INFINITY);
    }
    return SPARSEPR_OK;
}

int32_t sparsepr_get_stats(sparsepr_ctx* c, sparsepr_stats* out) {
    if (!c || !out) return SPARSEPR_ERR_INVALID_ARG;
    int32_t rc = enter(c, 0);
    if (rc) return rc;
    std::memset(out, 0, sizeof(*out));
    out->routed_k = c->k;
    out->query_dims = c->Dq;
    if (c->last_stream || c->stage > 0) SPR_HIP(c, hipStreamSynchronize(c->last_stream));
    if (c->stage >= kStageRoute) {
        std::vector<int64_t> pairs(c->H);
        SPR_HIP(c, hipMemcpy(pairs.data(), c->pairs, 8 * (size_t)c->H, hipMemcpyDeviceToHost));
        for (int64_t v : pairs) out->routed_pairs += v;
        out->probe_pairs = (int64_t)c->P * c->N * c->H;
        out->exec_density = (double)(out->routed_pairs + out->probe_pairs) /
                            ((double)c->H * (double)c->N * (double)c->N);
    }
    if (c->check_finite && c->stage >= kStagePartition) {
        unsigned long long nf[2] = {0, 0};
        SPR_HIP(c, hipMemcpy(nf, c->nonfinite, sizeof(nf), hipMemcpyDeviceToHost));
        out->nonfinite_inputs = (int64_t)nf[0];
        out->nonfinite_outputs = (int64_t)nf[1];
    }
    out->metric_gap_min = INFINITY;
    out->resid_gap_min = INFINITY;
    if (c->stage >= kStagePartition) {
        if (c->mgap_dev) SPR_HIP(c, hipMemcpy(c->h_mgap.data(), c->mgap, 8 * (size_t)c->H, hipMemcpyDeviceToHost));
        for (double g : c->h_mgap) out->metric_gap_min = std::min(out->metric_gap_min, g);
    }
    if (c->stage >= kStageFit)
        for (double g : c->h_rgap) out->resid_gap_min = std::min(out->resid_gap_min, g);
    if (c->stage >= kStagePartition) {
        std::vector<int32_t> fl(2 * (size_t)c->T * c->H);
        SPR_HIP(c, hipMemcpy(fl.data(), c->flag_cnt, 4 * fl.size(), hipMemcpyDeviceToHost));
        for (int32_t v : fl) out->recheck_points += v;
    }
    if (c->timing) {
        // average over the calls since the previous sparsepr_get_stats that the ring still holds
        const int pairs_ev[6][2] = {{0, 1}, {2, 3}, {4, 5}, {3, 4}, {5, 6}, {6, 7}};
        const int64_t first = std::max(c->stats_from, c->calls - sparsepr_ctx::kRing);
        for (int i = 0; i < 6; ++i) {
            double sum = 0.0;
            int cnt = 0;
            for (int64_t call = first; call < c->calls; ++call) {
                const int s = (int)(call % sparsepr_ctx::kRing);
                float ms = 0.f;
                if (c->ev_used[s][pairs_ev[i][0]] && c->ev_used[s][pairs_ev[i][1]] &&
                    hipEventElapsedTime(&ms, c->ev[s][pairs_ev[i][0]], c->ev[s][pairs_ev[i][1]]) == hipSuccess) {
                    sum += ms;
                    ++cnt;
                }
            }
            out->stage_ms[i] = cnt ? (float)(sum / cnt) : 0.f;
            if (i == 2) out->timed_calls = cnt;
        }
        c->stats_from = c->calls;
    }
    return SPARSEPR_OK;
}

// ------------------------------------------------------------- host solves ---
int32_t sparsepr_host_sym_eig_top(int32_t n, const double* a, int32_t r, double* lam, double* vec) {
    if (n < 1 || n > 1024 || r < 0 || r > n || !a || (r > 0 && (!lam || !vec))) return SPARSEPR_ERR_INVALID_ARG;
    return sym_eig_top(n, a, r, lam, vec) == 0 ? SPARSEPR_OK : SPARSEPR_ERR_NUMERIC;
}

int32_t sparsepr_host_key_projection(int32_t d, const double* m_k, int32_t r, double* w) {
    if (d < 1 || d > 1024 || r < 1 || r > d || !m_k || !w) return SPARSEPR_ERR_INVALID_ARG;
    return key_projection(d, m_k, r, w, nullptr) == 0 ? SPARSEPR_OK : SPARSEPR_ERR_NUMERIC;
}

int32_t sparsepr_host_probe_fit(int32_t p, int32_t d, const double* x, const double* y, double lambda,
                                int32_t rank, double* b_mat, double* b_vec) {
    if (p < 0 || d < 1 || d > 1024 || rank < 0 || rank > d || !(lambda >= 0.0) || !b_mat || !b_vec ||
        (p > 0 && (!x || !y)))
        return SPARSEPR_ERR_INVALID_ARG;
    return probe_fit(p, d, x, y, lambda, rank, b_mat, b_vec) == 0 ? SPARSEPR_OK : SPARSEPR_ERR_NUMERIC;
}

}  // extern "C"
