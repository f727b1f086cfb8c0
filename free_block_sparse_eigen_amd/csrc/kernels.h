// Launchers of the SparsePR HIP kernels (host-callable; all asynchronous on `st`).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

#include "common.h"

namespace spr {

constexpr int kSortChunk = 1024;      // points per counting-sort block
constexpr int kMaxGroups = 1024;      // G_k, G_q upper bound (LDS tables)
constexpr int kSparseRows = 128;      // query rows per sparse attention unit (4 waves, 2 blocks/CU)
constexpr int kDenseRows = 256;       // query rows per dense attention unit (8 waves, 1 block/CU)
constexpr int kKeyTile = 64;          // keys per attention tile
constexpr int kProbeRows = 256;       // probe rows per probe work unit (8 waves of 32)

// ---- generic ----
void launch_to_bf16(const float* in, bf16_t* out, size_t count, hipStream_t st);
void launch_fill_i32(int32_t* p, int32_t value, size_t count, hipStream_t st);
void launch_fill_i64(int64_t* p, int64_t value, size_t count, hipStream_t st);
// adds the number of non-finite values among x[0 .. count) (bf16, or fp32 if is_f32) to *counter
void launch_count_nonfinite(const void* x, size_t count, int is_f32, unsigned long long* counter,
                            hipStream_t st);

// ---- partition ----
constexpr int kEigMaxN = 128;         // device eigensolve: matrix order
constexpr int kEigMaxR = 64;          // device eigensolve: leading eigenvectors kept
// Leading r eigenpairs of the symmetric m [heads][n][n] (n <= kEigMaxN, r <= kEigMaxR) on the
// device: w [heads][n][r] = U_r diag(sqrt(max(lambda, 0))), gap [heads] = lambda_r/lambda_{r+1}
// (+inf if r = n or lambda_{r+1} <= 0). Scratch: diag, off, hbeta, tnorm [heads][n] (tnorm
// [heads]), hv [heads][n][n], lam [heads][r+1], vec [heads][r][n].
void launch_sym_eig_top(const double* m, int heads, int n, int r, double* diag, double* off,
                        double* hv, double* hbeta, double* lam, double* vec, double* tnorm,
                        double* w, double* gap, hipStream_t st);
void launch_metric(const bf16_t* q, int heads, int n, int d, int n_sample, int64_t a, double* mk,
                   hipStream_t st);
// The metric is a factor l64 [d][dout] (metric = L L^T), or with dout == 0 the full
// metric l64 [d][d]; c64 then holds the fp64 screening vectors M m ([groups][d]).
// raw centroids = the rows at the first `groups` Weyl indices (no screening tables)
void launch_seed_raw(const bf16_t* x, int heads, int n, int d, int groups, int64_t a, double* mean_raw,
                     hipStream_t st);
// screening tables of every centroid (empty groups included) from raw means and a metric
void launch_finish_all(const double* mean_raw, int heads, int d, const double* l64, int dout, int groups,
                       double* c64, bf16_t* cpart, float* cn2, float* cpn, double* c2_64, hipStream_t st,
                       double* crow = nullptr);
void launch_seed_centroids(const bf16_t* x, int heads, int n, int d, const double* l64, int dout,
                           int groups, int64_t a, double* mean_raw, double* c64, bf16_t* cpart,
                           float* cn2, float* cpn, double* c2_64, hipStream_t st, double* crow = nullptr,
                           int coords = 0);
void launch_assign(const bf16_t* x, int heads, int n, int d, const bf16_t* cpart, const float* cn2,
                   const float* cpn, int groups, int32_t* labels, int32_t* flag_count,
                   int32_t* flag_list, hipStream_t st, const bf16_t* zhl = nullptr, const float* kb = nullptr,
                   int dz = 0);
void launch_recheck(const bf16_t* x, int heads, int n, int d, const double* l64, int dim,
                    const double* c64, const double* c2_64, int groups, const int32_t* flag_count,
                    const int32_t* flag_list, int32_t* labels, hipStream_t st);
// Candidate lists for a long recheck queue when k_assign streams the centroids
// (assign_streams): cand [heads][n][kMaxCandidates], ncand [heads][n] by
// queue position (-1: too many, the point is queued in ovf_count/ovf_list [heads][n] for
// launch_recheck); then the fp64 recheck over them.
constexpr int kMaxCandidates = 32;
constexpr int kCandidateMaxDim = 32;     // factor widths above this take the full recheck
bool assign_streams(int groups, int d);
// zhl, kb, dz (the key side screened in its split coordinates, dz = r_K of 16 or 32): the
// queued keys are screened again in those coordinates against cpart's split coordinates
void launch_candidates(const bf16_t* x, int heads, int n, int d, const bf16_t* cpart, const float* cn2,
                       const float* cpn, int groups, const int32_t* flag_count, const int32_t* flag_list,
                       int32_t* cand, int32_t* ncand, int32_t* ovf_count, int32_t* ovf_list, hipStream_t st,
                       const bf16_t* zhl = nullptr, const float* kb = nullptr, int dz = 0);
void launch_recheck_cand(const bf16_t* x, int heads, int n, int d, const double* l64, int dim,
                         const double* crow, const double* c2_64, int groups, const int32_t* flag_count,
                         const int32_t* flag_list, const int32_t* cand, const int32_t* ncand,
                         const double* ycoord, int32_t* labels, hipStream_t st);
// every point's factor coordinates y = x L [heads][n][dim] (fp64) as the recheck forms them
void launch_coords(const bf16_t* x, int heads, int n, int d, const double* l64, int dim, double* y,
                   hipStream_t st);
// the same coordinates on MFMA for the screen in the key coordinates (launch_assign with
// zhl, kb; dim 16 or 32): zhl [heads][n][2][dim] bf16 (hi then lo), kb [heads][n] each
// point's bound coefficient
void launch_zcoords(const bf16_t* x, int heads, int n, int d, const double* l64, int dim, bf16_t* zhl,
                    float* kb, hipStream_t st);
void launch_counting_sort(const int32_t* labels, int heads, int n, int groups, int32_t* blkhist,
                          int32_t* blkoff, int32_t* sorted, int32_t* off, hipStream_t st);
void launch_group_means(const bf16_t* x, int heads, int n, int d, const int32_t* sorted,
                        const int32_t* off, int groups, double* mean_raw, const double* l64,
                        int dout, double* c64, bf16_t* cpart, float* cn2, float* cpn,
                        double* c2_64, hipStream_t st, double* crow = nullptr, int coords = 0);
// crow (optional): a row-major [heads][groups][d or dout] copy of the screening vectors
// (full metric) or of the centroid coordinates (factor) for the candidate recheck; coords
// (factor only): the assignment screens in the key coordinates (launch_assign with zhl), so
// the split centroid rows are the coordinates themselves ([heads][2][groups][dout])

// ---- route ----
void launch_permute(const bf16_t* src, const int32_t* perm, int heads, int n, int d, bf16_t* dst,
                    hipStream_t st);
// V into group-major fp16 scaled per head by 2^v_scale_exp(vmax[h]); vmax [heads] receives
// each head's largest |v| as bf16 magnitude bits
void launch_permute_v16(const bf16_t* src, const int32_t* perm, int heads, int n, int d,
                        uint32_t* vmax, uint16_t* dst, hipStream_t st);
// K into group-major FP8 E4M3 scaled per head by 2^f8_scale_exp(kmax[h]) (kmax [heads]: each
// head's largest |k| as bf16 magnitude bits, from launch_absmax_v); the fp8-logit experiment
void launch_permute_k8(const bf16_t* src, const int32_t* perm, int heads, int n, int d, const uint32_t* kmax,
                       uint8_t* dst, hipStream_t st);
// its two halves: the per-head magnitude bits, then the scaled permute that reads them
void launch_absmax_v(const bf16_t* src, int heads, int n, int d, uint32_t* vmax, hipStream_t st);
void launch_permute_f16(const bf16_t* src, const int32_t* perm, int heads, int n, int d,
                        const uint32_t* vmax, uint16_t* dst, hipStream_t st);
// ck_t: scratch [heads][d][gk] for the coordinate-major copy of ck
void launch_route(const double* cq, const double* ck, double* ck_t, const int32_t* qoff,
                  const int32_t* koff, int heads, int gq, int gk, int d, int k, int32_t* blocks,
                  int32_t* ucount, int64_t* pairs, hipStream_t st);
void launch_probes(const int32_t* qoff, const int32_t* qperm, int heads, int n, int gq, int probes,
                   int32_t* probe_pos, int32_t* probe_orig, int32_t* probe_grp, int32_t* probe_of,
                   hipStream_t st);
// units / nunits: rows_per_unit-row units; with big_rows > 0 each group's whole big_rows-row
// chunks go to units_big / nunits_big instead ([heads][max_big]) and only the rest of the
// group to units
void launch_units(const int32_t* qoff, int heads, int gq, int rows_per_unit, int max_units,
                  int2* units, int32_t* nunits, hipStream_t st, int big_rows = 0, int max_big = 0,
                  int2* units_big = nullptr, int32_t* nunits_big = nullptr);
// this thread's error detail for calls without a context (sparsepr_last_error(NULL))
void set_call_error(const char* msg);

// ---- attention ----
// out_mode 0: fp32 rows, 1: bf16 rows (both at the unit's own row index); unit_rows is
// kSparseRows or kDenseRows (the units' row count, which fixes the block shape: 4 or 8
// waves)
// qp: Q in token order; qperm [heads][n] (group-major position -> token) or nullptr
// vp: bf16 [heads][n][d] with vmax == nullptr (dense baseline), or fp16 scaled per head by
// 2^v_scale_exp(vmax[h]) (the sparse call); kp8 (128-row units only) (with qmax, kmax: the
// per-head largest |q| and |k| as bf16 magnitude bits) selects the fp8-logit experiment:
// K group-major in FP8 E4M3 scaled by 2^f8_scale_exp(kmax[h]), Q rounded on load
void launch_vbsa(const bf16_t* qp, const int32_t* qperm, const bf16_t* kp, const void* vp,
                 const uint32_t* vmax, int heads, int n, int d,
                 const int32_t* qoff, int qoff_stride, const int32_t* koff, int koff_stride,
                 const int32_t* blocks, int blocks_head_stride, int kblk, const int2* units,
                 int units_head_stride, const int32_t* nunits, int nunits_stride, int max_units,
                 int unit_rows, void* out, int out_mode, hipStream_t st, const uint8_t* kp8 = nullptr,
                 const uint32_t* qmax = nullptr, const uint32_t* kmax = nullptr);
int probe_splits(int n, int heads, int probes);
// qp: Q in token order, probe_orig: the probe rows' token indices; kp group-major
// vtok: bf16 V in token order, gathered through kperm [heads][n] (group-major -> token)
void launch_probe(const bf16_t* qp, const bf16_t* kp, const bf16_t* vtok, const int32_t* kperm,
                  int heads, int n, int d,
                  const int32_t* probe_orig, const int32_t* probe_grp, int probes,
                  const int32_t* koff, int koff_stride, int gk, const int32_t* blocks, int gq,
                  int kblk, int splits, float* part_ml, float* part_od, float* part_os,
                  hipStream_t st);
void launch_probe_merge(int heads, int probes, int d, int splits, const float* part_ml,
                        const float* part_od, const float* part_os, float* x, float* y, float* od,
                        hipStream_t st);

// ---- correction ----
void launch_correct(const float* o_s, const bf16_t* bt16, const float* bvec, const float* od,
                    const int32_t* probe_orig, const int32_t* qperm, int heads, int n, int d,
                    int probes, void* o, int out_f32, hipStream_t st);

// ---- fit Grams (fp64) ----
void launch_col_means_f32(const float* a, int heads, int p, int d, double* mean, hipStream_t st);
void launch_gram_f32(const float* a, const float* b, const double* ma, const double* mb, int heads,
                     int p, int d, double* out, hipStream_t st);
void launch_gram_f64(const double* a, int heads, int p, int d, double scale, double* out,
                     hipStream_t st);

}  // namespace spr
