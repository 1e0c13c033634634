// api.hip -- the extern "C" entry points declared in include/semicrf.h.
//
// Host side only: argument validation (before any launch), launch
// configuration, workspace carve-up and launch sequencing on the caller's
// stream.  No allocation, no synchronisation, no state between calls.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "../../include/semicrf.h"
#include "internal.h"

using namespace semicrf;

// Device scratch of semicrf_fwd_bwd_static (for callers that cannot
// allocate): a file-scope array each GPU holds once the library runs on it.
// Host code never uses this name as an address (it is a host-side stand-in);
// static_scratch() looks the device address up per device.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

// Pick the chain workgroup shape for (C, K): the smallest workgroup whose
// per-thread duration count fits the register arrays (32 at 256/512 threads,
// 16 at 1024), whose contraction slices fit, and whose LDS fits 160 KB.
bool chain_config(int C, int K, ChainShape &sh) {
  if (C < 1 || C > kMaxC || K < 1 || (long long)K * C > kMaxKC) return false;
  const int nts[3] = {256, 512, 1024};
  const int amax[3] = {32, 32, 16};
  const int Q = (C + 63) / 64;
  for (int i = 0; i < 3; ++i) {
    const int NT = nts[i];
    const int P = NT / C;
    // Q * C <= NT: contraction slices never straddle; (Q + 2) * 64 <= NT: at
    // least two waves hold no row thread (score loader and row writer roles)
    if (P < 1 || Q * C > NT || (Q + 2) * 64 > NT) continue;
    const int A = (K + P - 1) / P;
    if (A > amax[i]) continue;
    int QT, CS;
    chain_slices(C, NT, QT, CS);
    if (CS > kTrwRows) continue;  // the widest slice instance
    if (chain_lds_bytes(C, K, P, QT, 0) > kMaxDynLds) continue;
    if (viterbi_lds_bytes(C, K, P, Q) > kMaxDynLds) continue;
    // helper waves: enough row writers for the 2C logs of a step (two per
    // lane), the rest load scores; a prefetch block of up to 8 positions,
    // at most kMaxPairs (position, label) pairs per loader lane, in the LDS
    // left over (below 2 positions the rows load their scores themselves)
    const int helpers = NT / 64 - Q;
    int writers = (C + 63) / 64;
    writers = writers < 1 ? 1 : (writers > helpers - 1 ? helpers - 1 : writers);
    const int loaders = helpers - writers;
    int pf = kMaxPairs * 64 * loaders / C;
    pf = pf > 8 ? 8 : pf;
    while (pf > 0 && chain_lds_bytes(C, K, P, QT, pf) > kMaxDynLds) --pf;
    if (pf < 2) pf = 0;
    sh.NT = NT;
    sh.P = P;
    sh.A = A;
    sh.Q = Q;
    sh.QT = QT;
    sh.CS = CS;
    sh.pf = pf;
    sh.nload = loaders;
    return true;
  }
  return false;
}

// Blocked windowed engine (C <= 32, 256 threads): applies when its LDS (the
// ring, K*C float64, plus block buffers) fits and each helper thread's far
// durations fit its registers (at most 8 * kWinFarChunks).  Other shapes run
// on the LDS-ring engine.
bool win_config(int C, int K, ChainShape &sh) {
  if (C < 1 || C > 32) return false;
  const int NT = 256;
  int cp = 1;  // label lanes per duration group: C rounded up to a power of two
  while (cp < C) cp *= 2;
  // far parts: durations k >= 2U over the three helper waves
  const int P = (NT - 64) / cp;
  const int nfar = K - (2 * kWinU - 1);
  int A = nfar > 0 ? (nfar + P - 1) / P : 1;
  // a whole number of the far loop's duration chunks (2, 4 or 8) per group,
  // so no chunk reaches into the next group's durations
  const int dch = A <= 2 ? 2 : (A <= 4 ? 4 : 8);
  A = (A + dch - 1) / dch * dch;
  if (A > dch * (dch == 8 ? kWinFarChunks : 1)) return false;
  if (win_lds_bytes(C, K, P) > kMaxDynLds) return false;
  // wave 1's groups take A durations each; waves 2-3, which also write the
  // rows (a logarithm per lane and block, more than wave 1's score loads),
  // share what is left: at most A, a whole number of chunks
  const int gw = 64 / cp;  // duration groups per helper wave
  const int rem = nfar - gw * A;
  int A2 = rem > 0 ? (rem + 2 * gw - 1) / (2 * gw) : 0;
  A2 = (A2 + dch - 1) / dch * dch;
  sh.NT = NT;
  sh.P = P;
  sh.A = A;
  sh.A2 = A2;
  sh.Q = 1;
  sh.win = 1;
  return true;
}

semicrf_status_t check_sizes(int B, int T, int C, int K) {
  if (B < 1 || T < 1 || C < 1 || K < 1) return SEMICRF_ERR_SHAPE;
  if ((long long)B * (T + 1) * C >= (1LL << 31)) return SEMICRF_ERR_SHAPE;
  return SEMICRF_OK;
}

int default_delta(int T, int K) {
  double d = ceil(sqrt((double)T * (double)K));
  if (d < 1) d = 1;
  if (d > T) d = T;
  return (int)d;
}

// Interval used when the caller passes 0: the sqrt(T*K) rule, halved while
// the sweep (one workgroup per direction and interval) would have fewer
// workgroups than the chip holds at once -- each interval is a serial chain
// of its length, so more intervals finish sooner until the chip is full --
// and never below max(2K, 32) positions, so each interval spans several
// segment lengths and forgets its neutral start.  The chip holds one
// workgroup per compute unit of every engine, and two of the windowed
// engine while two of its LDS footprints fit one compute unit: one chain's
// step is a latency-bound dependent chain, and a second chain on the same
// unit hides most of it (measured at C = 16: 638 ns per step alone, 764 ns
// with two per unit).
constexpr long long kSweepWorkgroups = 256;

// Two windowed workgroups per compute unit need two LDS footprints and two
// waves' registers per SIMD (at most 256 VGPRs + AGPRs a wave): the
// instances for C <= 16 take 250, those for 16 < C <= 32 with far chunks of
// 8 durations 263 (one per unit), with chunks of 2 or 4 durations 209.
long long sweep_workgroups(int C, int K) {
  ChainShape w{};
  if (win_config(C, K, w) && (C <= 16 || w.A <= 4) &&
      2 * (win_lds_bytes(C, K, w.P) + 256) <= kMaxLds)
    return 2 * kSweepWorkgroups;
  return kSweepWorkgroups;
}

// Burn-in of a chunk without an exact start (parallel-in-time iteration 0),
// for intervals of at least 8K positions, or of at least 4K and 1024
// positions (the burn-in then costs at most 1/32 of the interval):
// kBurnIn positions.  The ring's
// entries are exp-space values relative to the newest ones, and the scores
// grow by several nats per position, so entries a few dozen positions old
// weigh nothing at the verification's 1e-12; what has to settle is the
// direction of the newest entries.  Measured: 32 positions converge in one
// iteration on the speech, genome and extreme workloads (a quarter of the
// interval cost up to 1024 extra positions per chunk).  A chunk that does
// not converge is swept again, so the result never depends on this choice.
// Shorter intervals (NLP-sized) sweep twice instead: there a burn-in that
// converges costs as much as the second sweep.
constexpr int kBurnIn = 32;

int burn_in(int delta, int K) {
  const long long d = delta;
  return (d >= 8LL * K || (d >= 4LL * K && d >= 32 * kBurnIn)) ? kBurnIn : 0;
}

int effective_delta(int B, int T, int C, int K) {
  int d = default_delta(T, K);
  const int dmin = 2 * K > 32 ? 2 * K : 32;
  const long long target = sweep_workgroups(C, K);
  while ((d + 1) / 2 >= dmin && 2LL * B * ((T + d - 1) / d) < target) d = (d + 1) / 2;
  return d;
}

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  }
};

// Low-memory posterior windows: ceil(sqrt(nchunk)) forward chunks per
// window, so the rows of a window (about sqrt(nchunk) * delta positions)
// grow like T^(3/4) K^(1/4) with the default interval: sublinear in T, as the
// records (nchunk rings of K x C) are.
int lowmem_window(int nchunk) {
  int w = 1;
  while (w * w < nchunk) ++w;
  return w;
}

// Workspace layout for an op.  Returns false for an invalid op.
bool make_layout(int op, int B, int T, int C, int K, const ChainShape *sh, Layout &lay,
                 const VShape *vs = nullptr) {
  Carver cv;
  lay = Layout{};
  lay.scan_j = scan_j(B, T, C);
  const int tile = scan_rows(C) * lay.scan_j;
  lay.ntile = (T + tile - 1) / tile;
  const size_t nS = (size_t)B * (T + 1) * C;
  if (op != SEMICRF_OP_SCAN) {
    lay.S = cv.take(nS * 8);
    lay.nu = cv.take((size_t)B * C * 8);
  }
  lay.tile_sum = cv.take((size_t)B * lay.ntile * C * 8);
  lay.anchor = cv.take((size_t)B * lay.ntile * C * 8);
  switch (op) {
    case SEMICRF_OP_SCAN:
      break;
    case SEMICRF_OP_LOGZ:
    case SEMICRF_OP_FWD_BWD: {
      const size_t nck = (size_t)B * sh->nchunk;
      const size_t rec = nck * (size_t)(K + 3) * C * 8;
      const bool bwd = op == SEMICRF_OP_FWD_BWD;
      lay.logz = cv.take((size_t)B * 8);
      lay.logz_bwd = cv.take((size_t)B * 8);
      lay.ck_fwd = cv.take(rec);
      lay.end_fwd = cv.take(rec);
      lay.ck_bwd = bwd ? cv.take(rec) : 0;
      lay.end_bwd = bwd ? cv.take(rec) : 0;
      lay.redo = cv.take(2 * nck * 4);
      lay.corr_i = cv.take(2 * nck * 8);
      lay.corr_f = cv.take(2 * nck * 8);
      lay.nbad = cv.take((size_t)sh->nchunk * 4);
      lay.lz_part = cv.take((size_t)2 * B * 8);
      lay.shift = cv.take(2 * nck * 8);
      if (!sh->win && !sh->e64 && !sh->e256 && sh->NT == 1024) lay.trw = cv.take(trw_floats(C, sh->QT) * 4);
      if (!bwd) break;
      // rows of every position, or (low memory) of one window of chunks
      const int rs = sh->lm_w ? (sh->lm_w + sh->lm_h) * sh->delta + 1 : T + 1;
      const size_t nR = (size_t)B * rs * C;
      lay.row_stride = rs;
      lay.row_a = cv.take(nR * 8);
      lay.row_u = cv.take(nR * 8);
      lay.row_v = cv.take(nR * 8);
      lay.row_b = cv.take(nR * 8);
      if (!sh->lm_w) lay.pos_shift = cv.take((size_t)2 * B * (T + 1) * 8);
      PostGeom g;
      post_geometry(*sh, g, sh->lm_w ? sh->lm_w * sh->delta : T);
      lay.cov_part = cv.take((size_t)B * g.cov_ntile * C * 8);
      lay.cov_part2 = cv.take((size_t)B * g.cov_ntile * C * 8);
      lay.cov_anchor = cv.take((size_t)B * g.cov_ntile * C * 8);
      lay.cov_mean = cv.take((size_t)B * C * 8);
      if (sh->lm_w) lay.cov_carry = cv.take((size_t)B * C * 8);
      lay.tx_part = cv.take((size_t)B * g.tx_nseg * C * C * 8);
      lay.dur_part = cv.take((size_t)B * g.dur_nspan * K * C * 8);
      break;
    }
    case SEMICRF_OP_PATH_SCORE:
      lay.p_score = cv.take((size_t)B * 8);
      lay.p_valid = cv.take((size_t)B * 4);
      lay.p_cnt = cv.take((size_t)B * ((size_t)C * C + (size_t)K * C + C) * 4);
      lay.p_lab = cv.take((size_t)B * T * 4);
      break;
    case SEMICRF_OP_VITERBI:
      // decisions of every position, or (low memory) of one window of chunks
      // and the chunk before it
      lay.bp = cv.take(vs && vs->lm_w ? (size_t)B * C * ((size_t)(vs->lm_w + 1) * vs->delta + 1) * 4
                                      : nS * 4);
      lay.vbest = cv.take((size_t)B * 8);
      lay.vcbest = cv.take((size_t)B * 4);
      if (vs) {  // parallel-in-time decoder
        const size_t nck = (size_t)B * vs->nchunk;
        lay.vit_pit = 1;
        lay.v_rr = cv.take(nck * K * C * 8);
        lay.v_re = cv.take(nck * K * C * 8);
        lay.v_corr = cv.take(nck * 8);
        lay.v_delta = cv.take(nck * 8);
        lay.v_redo = cv.take(nck * 4);
        lay.v_nbad = cv.take((size_t)kVitIters * 4);
        if (vs->lm_w) {  // the parallel backtrack over one window at a time
          const size_t wpos = (size_t)vs->lm_w * vs->delta;  // positions of a window
          const size_t wst = wpos + vs->delta + 1;           // with the chunk before it
          const size_t wsub = (wpos + vs->dbt - 1) / vs->dbt;
          lay.v_pred = cv.take((size_t)B * C * wst * 4);
          lay.v_lst_t = cv.take((size_t)B * wpos * 4);
          lay.v_lst_c = cv.take((size_t)B * wpos * 4);
          lay.v_mark = cv.take((size_t)B * wst * 4);
          lay.v_sub = cv.take((size_t)B * wsub * kVSubFields * 4);
          lay.v_node = cv.take((size_t)B * 3 * 4);
        } else {  // the parallel backtrack over the whole sequence
          lay.v_pred = cv.take(nS * 4);
          lay.v_lst_t = cv.take((size_t)B * T * 4);
          lay.v_lst_c = cv.take((size_t)B * T * 4);
          lay.v_mark = cv.take((size_t)B * (T + 1) * 4);
          lay.v_sub = cv.take((size_t)B * vs->nsub * kVSubFields * 4);
        }
      }
      break;
    default:
      return false;
  }
  lay.total = cv.off;
  return true;
}

// Validate sizes/flags and fill the shape + layout.  No launches.
semicrf_status_t prepare(int op, int B, int T, int C, int K, unsigned flags, int ckpt,
                         ChainShape &sh, Layout &lay, VShape *vs_out = nullptr) {
  if (op < SEMICRF_OP_SCAN || op > SEMICRF_OP_PATH_SCORE) return SEMICRF_ERR_ARG;
  if (flags & ~(unsigned)(SEMICRF_NO_CENTER | SEMICRF_LOW_MEMORY | SEMICRF_FLOAT64))
    return SEMICRF_ERR_ARG;
  if (ckpt < 0) return SEMICRF_ERR_ARG;
  const semicrf_status_t s = check_sizes(B, T, C, op == SEMICRF_OP_SCAN ? 1 : K);
  if (s != SEMICRF_OK) return s;
  if (C > kMaxC) return SEMICRF_ERR_UNSUPPORTED;
  sh = ChainShape{};
  sh.B = B;
  sh.T = T;
  sh.C = C;
  sh.K = K;
  sh.center = (flags & SEMICRF_NO_CENTER) ? 0 : 1;
  if (op != SEMICRF_OP_SCAN && op != SEMICRF_OP_PATH_SCORE) {
    // Viterbi always uses the LDS-ring layout; the sweeps use the windowed
    // engine when it applies.  Both must exist for a supported (C, K).
    ChainShape probe = sh;
    if (!chain_config(C, K, probe)) return SEMICRF_ERR_UNSUPPORTED;
    if (op == SEMICRF_OP_VITERBI || !win_config(C, K, sh)) sh = probe;
    // 32 < C <= 64 with K <= 256: the register-ring engine (chain64.hip)
    if (op != SEMICRF_OP_VITERBI && !sh.win && sweep64_applies(C, K)) sh.e64 = 1;
    // 64 < C <= 256 with K <= 64: the float32 wave-sliced contraction engine
    // (chain256.hip), unless the caller asks for float64 sweeps
    if (op != SEMICRF_OP_VITERBI && !sh.win && !sh.e64 && !(flags & SEMICRF_FLOAT64) &&
        sweep256_applies(C, K))
      sh.e256 = 1;
    const bool lowmem = op == SEMICRF_OP_FWD_BWD && (flags & SEMICRF_LOW_MEMORY);
    if (lowmem) {
      // the pages' interval (no splitting for parallelism: the records are
      // the working memory), at least K so one more backward chunk covers
      // the durations that reach past a window
      int d = ckpt > 0 ? ckpt : default_delta(T, K);
      if (d < K) d = K;
      sh.delta = d < T ? d : T;
    } else {
      sh.delta = ckpt > 0 ? (ckpt < T ? ckpt : T) : effective_delta(B, T, C, K);
    }
    sh.nchunk = (T + sh.delta - 1) / sh.delta;
    sh.burn = burn_in(sh.delta, K);
    if (lowmem) {
      sh.lm_w = lowmem_window(sh.nchunk);
      sh.lm_h = sh.nchunk > sh.lm_w ? 1 : 0;  // delta >= K: one chunk past the window
    }
  }
  VShape vs;
  const bool pit = op == SEMICRF_OP_VITERBI && vit_config(B, T, C, K, vs);
  if (pit) vs.center = sh.center;
  // low-memory decoding: decisions recomputed window by window from the
  // chunk start states (ceil(sqrt(#chunks)) chunks a window)
  if (pit && (flags & SEMICRF_LOW_MEMORY) && vs.nchunk > 1) vs.lm_w = lowmem_window(vs.nchunk);
  if (!make_layout(op, B, T, C, K, &sh, lay, pit ? &vs : nullptr)) return SEMICRF_ERR_ARG;
  if (pit && vs_out) *vs_out = vs;
  return SEMICRF_OK;
}

template <typename P>
P *at(void *ws, size_t off) {
  return reinterpret_cast<P *>(static_cast<unsigned char *>(ws) + off);
}

Escaled escaled(void *ws, const Layout &lay) {
  Escaled es;
  es.S = at<double>(ws, lay.S);
  return es;
}

PitBufs pit_bufs(void *ws, const Layout &lay, bool bwd) {
  PitBufs pb;
  pb.ck_fwd = at<double>(ws, lay.ck_fwd);
  pb.end_fwd = at<double>(ws, lay.end_fwd);
  pb.ck_bwd = bwd ? at<double>(ws, lay.ck_bwd) : nullptr;
  pb.end_bwd = bwd ? at<double>(ws, lay.end_bwd) : nullptr;
  pb.redo = at<int>(ws, lay.redo);
  pb.corr_i = at<long long>(ws, lay.corr_i);
  pb.corr_f = at<double>(ws, lay.corr_f);
  pb.nbad = at<int>(ws, lay.nbad);
  pb.lz_part = at<double>(ws, lay.lz_part);
  pb.shift = at<double>(ws, lay.shift);
  pb.row_a = bwd ? at<double>(ws, lay.row_a) : nullptr;
  pb.row_u = bwd ? at<double>(ws, lay.row_u) : nullptr;
  pb.row_v = bwd ? at<double>(ws, lay.row_v) : nullptr;
  pb.row_b = bwd ? at<double>(ws, lay.row_b) : nullptr;
  pb.pos_shift = bwd && lay.pos_shift ? at<double>(ws, lay.pos_shift) : nullptr;
  pb.row_t0 = 0;
  pb.row_stride = lay.row_stride;
  pb.trw = lay.trw ? at<float>(ws, lay.trw) : nullptr;
  return pb;
}

// The device address of `scratch` on the current device: looked up with
// hipGetSymbolAddress on the first call with that device current, then
// reused (each GPU holds its own copy of the array at its own address).
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

hipError_t static_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// With SEMICRF_DEBUG set in the environment, name the HIP error on stderr.
semicrf_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return SEMICRF_OK;
  if (getenv("SEMICRF_DEBUG")) fprintf(stderr, "semicrf: HIP error %d: %s\n", (int)e, hipGetErrorString(e));
  return SEMICRF_ERR_HIP;
}

}  // namespace

extern "C" {

const char *semicrf_status_string(semicrf_status_t status) {
  switch (status) {
    case SEMICRF_OK: return "ok";
    case SEMICRF_ERR_NULL: return "a required pointer is NULL";
    case SEMICRF_ERR_SHAPE: return "invalid sizes (B, T, C, K must be >= 1; B*(T+1)*C < 2^31)";
    case SEMICRF_ERR_UNSUPPORTED: return "unsupported C or K (see semicrf.h)";
    case SEMICRF_ERR_WORKSPACE: return "workspace NULL or smaller than semicrf_workspace_size";
    case SEMICRF_ERR_HIP: return "HIP launch failed";
    case SEMICRF_ERR_ARG: return "invalid op, flags or checkpoint interval";
    case SEMICRF_ERR_SCRATCH:
      return "these sizes need more workspace than the 64 MiB static scratch of "
             "semicrf_fwd_bwd_static";
  }
  return "unknown status";
}

int semicrf_default_checkpoint_interval(int T, int K) {
  if (T < 1 || K < 1) return 0;
  return default_delta(T, K);
}

int semicrf_checkpoint_interval(int B, int T, int C, int K) {
  if (B < 1 || T < 1 || C < 1 || K < 1) return 0;
  return effective_delta(B, T, C, K);
}

semicrf_status_t semicrf_workspace_size(int op, int B, int T, int C, int K, unsigned flags,
                                        int checkpoint_interval, size_t *bytes) {
  if (!bytes) return SEMICRF_ERR_NULL;
  ChainShape sh;
  Layout lay;
  const semicrf_status_t s =
      prepare(op, B, T, C, K, flags, op == SEMICRF_OP_FWD_BWD ? checkpoint_interval : 0, sh, lay);
  if (s != SEMICRF_OK) return s;
  *bytes = lay.total;
  return SEMICRF_OK;
}

semicrf_status_t semicrf_cumulative_scores(const float *emissions, const int32_t *lengths, int B,
                                           int T, int C, unsigned flags, double *nu, double *S,
                                           void *workspace, size_t workspace_bytes,
                                           void *stream) {
  if (!emissions || !lengths || !nu || !S) return SEMICRF_ERR_NULL;
  ChainShape sh;
  Layout lay;
  const semicrf_status_t s = prepare(SEMICRF_OP_SCAN, B, T, C, 1, flags, 0, sh, lay);
  if (s != SEMICRF_OK) return s;
  if (!workspace || workspace_bytes < lay.total) return SEMICRF_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  return hip_status(launch_scan(emissions, lengths, B, T, C, sh.center, nu, S, nullptr,
                                nullptr, nullptr, at<double>(workspace, lay.tile_sum),
                                at<double>(workspace, lay.anchor), lay.ntile, lay.scan_j, st));
}

semicrf_status_t semicrf_logz_fwd(const float *emissions, const int32_t *lengths,
                                  const float *trans, const float *dur, int B, int T, int C, int K,
                                  unsigned flags, float *logz, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  if (!emissions || !lengths || !trans || !dur || !logz) return SEMICRF_ERR_NULL;
  ChainShape sh;
  Layout lay;
  const semicrf_status_t s = prepare(SEMICRF_OP_LOGZ, B, T, C, K, flags, 0, sh, lay);
  if (s != SEMICRF_OK) return s;
  if (!workspace || workspace_bytes < lay.total) return SEMICRF_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  double *S = at<double>(workspace, lay.S);
  const Escaled es = escaled(workspace, lay);
  hipError_t e = launch_scan(emissions, lengths, B, T, C, sh.center, at<double>(workspace, lay.nu),
                             S, nullptr, nullptr, nullptr, at<double>(workspace, lay.tile_sum),
                             at<double>(workspace, lay.anchor), lay.ntile, lay.scan_j, st);
  if (e != hipSuccess) return hip_status(e);
  e = run_sweeps(sh, trans, dur, es, lengths, pit_bufs(workspace, lay, false),
                 at<double>(workspace, lay.logz), nullptr, logz, 0, st);
  return hip_status(e);
}

semicrf_status_t semicrf_fwd_bwd_ex(const float *emissions, const int32_t *lengths,
                                    const float *trans, const float *dur, int B, int T, int C,
                                    int K, unsigned flags, int checkpoint_interval,
                                    const float *grad_logz, float *logz, float *grad_emissions,
                                    float *grad_trans, float *grad_dur, float *marginals,
                                    float *boundary, void *workspace, size_t workspace_bytes,
                                    void *stream, void *const *phase_events) {
  if (!emissions || !lengths || !trans || !dur || !logz || !grad_emissions || !grad_trans ||
      !grad_dur)
    return SEMICRF_ERR_NULL;
  ChainShape sh;
  Layout lay;
  const semicrf_status_t s =
      prepare(SEMICRF_OP_FWD_BWD, B, T, C, K, flags, checkpoint_interval, sh, lay);
  if (s != SEMICRF_OK) return s;
  if (!workspace || workspace_bytes < lay.total) return SEMICRF_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  auto mark = [&](int i) {
    if (phase_events) (void)hipEventRecord(static_cast<hipEvent_t>(phase_events[i]), st);
  };
  void *ws = workspace;
  double *S = at<double>(ws, lay.S);
  mark(0);
  hipError_t e = launch_scan(emissions, lengths, B, T, C, sh.center, at<double>(ws, lay.nu), S,
                             nullptr, nullptr, nullptr, at<double>(ws, lay.tile_sum),
                             at<double>(ws, lay.anchor), lay.ntile, lay.scan_j, st);
  if (e != hipSuccess) return hip_status(e);
  mark(1);
  const bool lowmem = sh.lm_w > 0;
  PitBufs pb = pit_bufs(ws, lay, true);
  if (lowmem) {  // the sweeps keep the checkpoint records only
    pb.row_a = pb.row_u = pb.row_v = pb.row_b = nullptr;
  }
  e = run_sweeps(sh, trans, dur, escaled(ws, lay), lengths, pb, at<double>(ws, lay.logz),
                 at<double>(ws, lay.logz_bwd), logz, 1, st,
                 phase_events ? static_cast<hipEvent_t>(phase_events[2]) : nullptr);
  if (e != hipSuccess) return hip_status(e);
  mark(3);
  PostArgs pa;
  pa.lengths = lengths;
  pa.trans = trans;
  pa.dur = dur;
  pa.grad_logz = grad_logz;
  pa.S = S;
  pa.logz = at<double>(ws, lay.logz);
  pa.row_a = at<double>(ws, lay.row_a);
  pa.row_u = at<double>(ws, lay.row_u);
  pa.row_v = at<double>(ws, lay.row_v);
  pa.row_b = at<double>(ws, lay.row_b);
  pa.pos_shift = lay.pos_shift ? at<double>(ws, lay.pos_shift) : nullptr;
  pa.t_lo = 0;
  pa.t_hi = T;
  pa.row_t0 = 0;
  pa.row_stride = lay.row_stride;
  pa.geom_T = lowmem ? sh.lm_w * sh.delta : T;
  pa.accumulate = 0;
  pa.defer_mean = 0;
  pa.cov_carry = lay.cov_carry ? at<double>(ws, lay.cov_carry) : nullptr;
  pa.cov_part = at<double>(ws, lay.cov_part);
  pa.cov_part2 = at<double>(ws, lay.cov_part2);
  pa.cov_anchor = at<double>(ws, lay.cov_anchor);
  pa.cov_mean = at<double>(ws, lay.cov_mean);
  pa.tx_part = at<double>(ws, lay.tx_part);
  pa.dur_part = at<double>(ws, lay.dur_part);
  pa.grad_emissions = grad_emissions;
  pa.marginals = marginals;
  pa.grad_trans = grad_trans;
  pa.grad_dur = grad_dur;
  pa.boundary = boundary;
  if (!lowmem) {
    e = launch_posteriors(sh, pa, st);
    if (e != hipSuccess) return hip_status(e);
  } else {
    // windows of lm_w checkpoint intervals, in order: replay the window's
    // intervals (and lm_h more backward ones) from their exact records into
    // the row buffers, then the window's posteriors, which continue the
    // coverage sum and add to the partials of the windows before
    const Escaled es = escaled(ws, lay);
    PitBufs rb = pit_bufs(ws, lay, true);
    pa.defer_mean = 1;
    for (int j0 = 0, w = 0; j0 < sh.nchunk; j0 += sh.lm_w, ++w) {
      ChainShape rs = sh;
      rs.rj0 = j0;
      rs.rnf = sh.lm_w < sh.nchunk - j0 ? sh.lm_w : sh.nchunk - j0;
      rs.rnb = sh.lm_w + sh.lm_h < sh.nchunk - j0 ? sh.lm_w + sh.lm_h : sh.nchunk - j0;
      rb.row_t0 = j0 * sh.delta;
      e = launch_sweep(rs, trans, dur, es, lengths, rb, 1, -1, st);
      if (e != hipSuccess) return hip_status(e);
      pa.t_lo = j0 * sh.delta;
      pa.t_hi = (j0 + rs.rnf) * sh.delta < T ? (j0 + rs.rnf) * sh.delta : T;
      pa.row_t0 = pa.t_lo;
      pa.accumulate = w > 0;
      e = launch_posteriors(sh, pa, st);
      if (e != hipSuccess) return hip_status(e);
    }
    e = launch_mean_fix(sh, pa, st);
    if (e != hipSuccess) return hip_status(e);
  }
  mark(4);
  e = launch_post_reduce(sh, pa, st);
  if (e != hipSuccess) return hip_status(e);
  mark(SEMICRF_FWD_BWD_PHASES);
  return SEMICRF_OK;
}

semicrf_status_t semicrf_fwd_bwd(const float *emissions, const int32_t *lengths,
                                 const float *trans, const float *dur, int B, int T, int C, int K,
                                 unsigned flags, int checkpoint_interval, const float *grad_logz,
                                 float *logz, float *grad_emissions, float *grad_trans,
                                 float *grad_dur, float *marginals, void *workspace,
                                 size_t workspace_bytes, void *stream) {
  return semicrf_fwd_bwd_ex(emissions, lengths, trans, dur, B, T, C, K, flags,
                            checkpoint_interval, grad_logz, logz, grad_emissions, grad_trans,
                            grad_dur, marginals, nullptr, workspace, workspace_bytes, stream,
                            nullptr);
}

semicrf_status_t semicrf_fwd_bwd_static(const float *emissions, const int32_t *lengths,
                                        const float *trans, const float *dur, int B, int T,
                                        int C, int K, unsigned flags, int checkpoint_interval,
                                        const float *grad_logz, float *logz,
                                        float *grad_emissions, float *grad_trans,
                                        float *grad_dur, float *marginals, void *stream) {
  if (!emissions || !lengths || !trans || !dur || !logz || !grad_emissions || !grad_trans ||
      !grad_dur)
    return SEMICRF_ERR_NULL;
  ChainShape sh;
  Layout lay;
  const semicrf_status_t s =
      prepare(SEMICRF_OP_FWD_BWD, B, T, C, K, flags, checkpoint_interval, sh, lay);
  if (s != SEMICRF_OK) return s;
  if (lay.total > kStaticScratchBytes) return SEMICRF_ERR_SCRATCH;
  void *ws = nullptr;
  const hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return hip_status(e);
  // every kernel of the call writes the workspace before it reads it, so
  // what an earlier call left there is never used
  return semicrf_fwd_bwd_ex(emissions, lengths, trans, dur, B, T, C, K, flags,
                            checkpoint_interval, grad_logz, logz, grad_emissions, grad_trans,
                            grad_dur, marginals, nullptr, ws, kStaticScratchBytes, stream,
                            nullptr);
}

semicrf_status_t semicrf_path_score(const float *emissions, const int32_t *lengths,
                                    const float *trans, const float *dur, int B, int T, int C,
                                    int K, unsigned flags, const int32_t *seg_start,
                                    const int32_t *seg_len, const int32_t *seg_label,
                                    const int32_t *num_segs, const float *weights, float *score,
                                    float *grad_emissions, float *grad_trans, float *grad_dur,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  if (!emissions || !lengths || !trans || !dur || !seg_start || !seg_len || !seg_label ||
      !num_segs || !score)
    return SEMICRF_ERR_NULL;
  ChainShape sh;
  Layout lay;
  const semicrf_status_t s = prepare(SEMICRF_OP_PATH_SCORE, B, T, C, K, flags, 0, sh, lay);
  if (s != SEMICRF_OK) return s;
  if (!workspace || workspace_bytes < lay.total) return SEMICRF_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  void *ws = workspace;
  double *S = at<double>(ws, lay.S);
  hipError_t e = launch_scan(emissions, lengths, B, T, C, sh.center, at<double>(ws, lay.nu), S,
                             nullptr, nullptr, nullptr, at<double>(ws, lay.tile_sum),
                             at<double>(ws, lay.anchor), lay.ntile, lay.scan_j, st);
  if (e != hipSuccess) return hip_status(e);
  PathArgs pa;
  pa.lengths = lengths;
  pa.trans = trans;
  pa.dur = dur;
  pa.w = weights;
  pa.S = S;
  pa.seg_start = seg_start;
  pa.seg_len = seg_len;
  pa.seg_label = seg_label;
  pa.num_segs = num_segs;
  pa.score = score;
  pa.grad_x = grad_emissions;
  pa.grad_trans = grad_trans;
  pa.grad_dur = grad_dur;
  pa.score_ws = at<double>(ws, lay.p_score);
  pa.valid = at<int>(ws, lay.p_valid);
  pa.cnt = at<int>(ws, lay.p_cnt);
  pa.lab = at<int32_t>(ws, lay.p_lab);
  return hip_status(launch_path_score(sh, pa, st));
}

semicrf_status_t semicrf_viterbi(const float *emissions, const int32_t *lengths,
                                 const float *trans, const float *dur, int B, int T, int C, int K,
                                 unsigned flags, float *best_score, int32_t *seg_start,
                                 int32_t *seg_len, int32_t *seg_label, int32_t *num_segs,
                                 void *workspace, size_t workspace_bytes, void *stream) {
  if (!emissions || !lengths || !trans || !dur || !best_score || !seg_start || !seg_len ||
      !seg_label || !num_segs)
    return SEMICRF_ERR_NULL;
  ChainShape sh;
  Layout lay;
  VShape vs;
  const semicrf_status_t s = prepare(SEMICRF_OP_VITERBI, B, T, C, K, flags, 0, sh, lay, &vs);
  if (s != SEMICRF_OK) return s;
  if (K > 65535 || C > 65535) return SEMICRF_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < lay.total) return SEMICRF_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  void *ws = workspace;
  double *S = at<double>(ws, lay.S);
  hipError_t e = launch_scan(emissions, lengths, B, T, C, sh.center, at<double>(ws, lay.nu), S,
                             nullptr, nullptr, nullptr, at<double>(ws, lay.tile_sum),
                             at<double>(ws, lay.anchor), lay.ntile, lay.scan_j, st);
  if (e != hipSuccess) return hip_status(e);
  if (lay.vit_pit) {
    VBufs vb;
    auto opt = [&](size_t off) { return off ? at<int32_t>(ws, off) : nullptr; };
    vb.bp = at<uint32_t>(ws, lay.bp);
    vb.pred = lay.v_pred ? at<uint32_t>(ws, lay.v_pred) : nullptr;
    vb.rec_r = at<double>(ws, lay.v_rr);
    vb.rec_e = at<double>(ws, lay.v_re);
    vb.corr = at<double>(ws, lay.v_corr);
    vb.delta = at<double>(ws, lay.v_delta);
    vb.redo = at<int>(ws, lay.v_redo);
    vb.nbad = at<int>(ws, lay.v_nbad);
    vb.vbest = at<double>(ws, lay.vbest);
    vb.vcbest = at<int32_t>(ws, lay.vcbest);
    vb.lst_t = opt(lay.v_lst_t);
    vb.lst_c = opt(lay.v_lst_c);
    vb.mark = opt(lay.v_mark);
    vb.sub = opt(lay.v_sub);
    vb.node = opt(lay.v_node);
    e = launch_vit_pit(vs, trans, dur, S, lengths, vb, best_score, seg_start, seg_len,
                       seg_label, num_segs, st);
  } else {
    e = launch_viterbi(sh, trans, dur, S, lengths, at<uint32_t>(ws, lay.bp),
                       at<double>(ws, lay.vbest), at<int32_t>(ws, lay.vcbest), best_score,
                       seg_start, seg_len, seg_label, num_segs, st);
  }
  return hip_status(e);
}

}  // extern "C"
