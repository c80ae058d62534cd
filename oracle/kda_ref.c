/*
 * kda_ref.c -- the oracle: a plain, slow, sequential fp64 CPU loop of the
 * Kimi Delta Attention (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * constant with the HIP path and includes nothing from it.
 *
 * What it computes (state S in the key-by-value orientation, S is d_k x d_v,
 * row i = key channel, column j = value channel):
 *
 *   a      = exp(g_t)                       per key channel (g_t = log alpha_t)
 *   Sbar   = Diag(a) S_{t-1}                forget: decay key rows first
 *   p      = Sbar^T k_t                     predict
 *   e      = beta_t (v_t - p)               correct
 *   S_t    = Sbar + k_t e^T                 write
 *   o_t    = S_t^T (scale * q_t)            read after the write
 *
 * Sources:
 *  - "Kimi Unveils Delta Attention and K3 Architecture Updates", section 4
 *    (Kimi Delta Attention): the forget / predict / correct / write / read list,
 *    and the five-line reference recurrence in the transposed d_k x d_v layout
 *    with g = log alpha and retention exp(g).
 *  - "Kimi Delta Attention: Channel-Wise Memory Control", section "Change one
 *    piece of Gated DeltaNet" (the equation with S in R^{d_k x d_v}, decay by
 *    left multiplication of Diag(alpha)) and "The core update in a few lines".
 *  - "Linear Attention, From Scratch to Kimi 3", section 9 (cu_seqlens): packed
 *    requests never share recurrent state.
 *
 * Optional input transforms (kdaref_forward_ex, flags), each applied to the
 * raw inputs of a token before the step, in fp64:
 *  - KDAREF_L2NORM: q <- q / sqrt(sum q^2 + 1e-6), the same for k, per (token,
 *    head) vector ("Linear Attention, From Scratch to Kimi 3", section 7: each
 *    head's q and k are L2-normalised before the recurrence);
 *  - KDAREF_BETA_SIGMOID: beta <- 1 / (1 + exp(-beta)) (same page, section 6:
 *    the update strength is a sigmoid of a raw projection);
 *  - KDAREF_GATE: g <- -5 sigmoid(exp(A_log[h]) (g + bias[h, i])) (same page,
 *    section 6: a sigmoid scaled by -5 gives a log-retention in (-5, 0), from
 *    the projection, a per-channel bias and one sensitivity per head; the
 *    composition inside the sigmoid is this implementation's reading).
 *
 * With delta_rule == 0 the correction is replaced by e = beta_t v_t, i.e. the
 * delta term is removed.  With alpha == 1 and beta == 1 that is plain causal
 * linear attention ("Kimi Unveils ...", section 1.1).  This mode exists only
 * so that tests can pin the loop structure against the quadratic closed form.
 *
 * Numerics: every input is upcast exactly to double; no blocking, no
 * reordering; sums run over the key index in ascending order.  Build with
 * -O2 -ffp-contract=off and without fast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KDAREF_IO_F32 0
#define KDAREF_IO_BF16 1

#define KDAREF_L2NORM 1
#define KDAREF_BETA_SIGMOID 2
#define KDAREF_GATE 4
#define KDAREF_NORM_EPS 1e-6

/* Exact bf16 -> double: a bf16 value is the top 16 bits of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load_io(const void* base, int dtype, size_t idx) {
  if (dtype == KDAREF_IO_BF16) return bf16_bits_to_double(((const uint16_t*)base)[idx]);
  return (double)((const float*)base)[idx];
}

typedef struct {
  const void *q, *k, *v;
  int dtype;
  const float *g, *beta;
  const double* S0;
  const int32_t* cu_seqlens; /* NULL: batched [B,T,H,d]; else packed [T_total,H,d] */
  int B, T, H, dk, dv;
  double scale;
  int delta_rule;
  int flags;
  const float *A_log, *gate_bias; /* [H], [H, dk] (NULL: zero bias) */
  const int32_t* chains;
  const int64_t* out_offset; /* first output row of each selected chain */
  int n_chains;
  double* out;
  double* S_final;
  /* work queue */
  pthread_mutex_t lock;
  int next;
} job_t;

/* One chain (sequence n, head h): the token loop, strictly sequential. */
static void run_chain(const job_t* jb, int ci) {
  const int chain = jb->chains[ci];
  const int n = chain / jb->H, h = chain % jb->H;
  const int dk = jb->dk, dv = jb->dv, H = jb->H;
  int64_t row0, len;
  if (jb->cu_seqlens) {
    row0 = jb->cu_seqlens[n];
    len = (int64_t)jb->cu_seqlens[n + 1] - jb->cu_seqlens[n];
  } else {
    row0 = (int64_t)n * jb->T;
    len = jb->T;
  }
  double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
  double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
  double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
  double* a = (double*)malloc(sizeof(double) * (size_t)dk);
  double* vt = (double*)malloc(sizeof(double) * (size_t)dv);
  double* p = (double*)malloc(sizeof(double) * (size_t)dv);
  double* e = (double*)malloc(sizeof(double) * (size_t)dv);

  if (jb->S0) {
    memcpy(S, jb->S0 + (size_t)chain * dk * dv, sizeof(double) * (size_t)dk * dv);
  } else {
    memset(S, 0, sizeof(double) * (size_t)dk * dv);
  }

  double* out_rows = jb->out + (size_t)jb->out_offset[ci] * dv;
  for (int64_t t = 0; t < len; ++t) {
    const size_t tok = (size_t)(row0 + t);
    const size_t kbase = (tok * H + h) * (size_t)dk;
    const size_t vbase = (tok * H + h) * (size_t)dv;
    double nk = 1.0, nq = 1.0;  /* 1 / L2 norms (KDAREF_L2NORM) */
    if (jb->flags & KDAREF_L2NORM) {
      double sk = 0.0, sq = 0.0;
      for (int i = 0; i < dk; ++i) {
        const double x = load_io(jb->k, jb->dtype, kbase + i);
        const double y = load_io(jb->q, jb->dtype, kbase + i);
        sk += x * x;
        sq += y * y;
      }
      nk = 1.0 / sqrt(sk + KDAREF_NORM_EPS);
      nq = 1.0 / sqrt(sq + KDAREF_NORM_EPS);
    }
    for (int i = 0; i < dk; ++i) {
      kt[i] = load_io(jb->k, jb->dtype, kbase + i) * nk;
      qt[i] = jb->scale * (load_io(jb->q, jb->dtype, kbase + i) * nq);
      double gi = (double)jb->g[kbase + i];
      if (jb->flags & KDAREF_GATE) {
        const double bias = jb->gate_bias ? (double)jb->gate_bias[(size_t)h * dk + i] : 0.0;
        const double x = exp((double)jb->A_log[h]) * (gi + bias);
        gi = -5.0 / (1.0 + exp(-x));
      }
      a[i] = exp(gi);
    }
    for (int j = 0; j < dv; ++j) vt[j] = load_io(jb->v, jb->dtype, vbase + j);
    double b = (double)jb->beta[tok * H + h];
    if (jb->flags & KDAREF_BETA_SIGMOID) b = 1.0 / (1.0 + exp(-b));

    /* forget: Sbar = Diag(a) S (key rows) */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a[i];
    /* predict: p = Sbar^T k */
    for (int j = 0; j < dv; ++j) p[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) p[j] += S[(size_t)i * dv + j] * kt[i];
    /* correct */
    for (int j = 0; j < dv; ++j) e[j] = jb->delta_rule ? b * (vt[j] - p[j]) : b * vt[j];
    /* write: S = Sbar + k e^T */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * e[j];
    /* read after the write: o = S^T (scale q) */
    double* o = out_rows + (size_t)t * dv;
    for (int j = 0; j < dv; ++j) o[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) o[j] += S[(size_t)i * dv + j] * qt[i];
  }
  if (jb->S_final)
    memcpy(jb->S_final + (size_t)ci * dk * dv, S, sizeof(double) * (size_t)dk * dv);
  free(S); free(kt); free(qt); free(a); free(vt); free(p); free(e);
}

static void* worker(void* arg) {
  job_t* jb = (job_t*)arg;
  for (;;) {
    pthread_mutex_lock(&jb->lock);
    int ci = jb->next++;
    pthread_mutex_unlock(&jb->lock);
    if (ci >= jb->n_chains) break;
    run_chain(jb, ci);
  }
  return NULL;
}

/*
 * kdaref_forward: run the recurrence for the selected chains.
 *
 *  q, k      [rows, H, dk] in dtype (0 = fp32, 1 = bf16 bit patterns)
 *  v         [rows, H, dv] in dtype
 *  g         [rows, H, dk] fp32, g = log alpha (natural log)
 *  beta      [rows, H] fp32
 *  S0        [n_seq, H, dk, dv] fp64 or NULL (zeros)
 *  cu_seqlens NULL (batched: rows = B*T, sequence n covers rows n*T .. n*T+T-1)
 *            or [B+1] int32 boundary offsets (packed: B sequences, T = T_total)
 *  chains    [n_chains] chain ids n*H + h to compute (any order, no repeats)
 *  out       concatenation over the selected chains, in the order given, of
 *            each chain's [len, dv] outputs (fp64)
 *  S_final   [n_chains, dk, dv] fp64 or NULL
 *  threads   worker threads over independent chains (<= 0: 1)
 *  flags     KDAREF_* input transforms (0: none); g and beta then hold the
 *            raw projections they transform
 *  A_log     [H] fp32, required with KDAREF_GATE
 *  gate_bias [H, dk] fp32 or NULL (zero), with KDAREF_GATE
 * Returns 0, or -1 on bad arguments.
 */
int kdaref_forward_ex(const void* q, const void* k, const void* v, int dtype,
                      const float* g, const float* beta, const double* S0,
                      const int32_t* cu_seqlens, int B, int T, int H, int dk, int dv,
                      double scale, int delta_rule, int flags, const float* A_log,
                      const float* gate_bias, const int32_t* chains, int n_chains, double* out,
                      double* S_final, int threads) {
  if (!q || !k || !v || !g || !beta || !chains || !out) return -1;
  if ((flags & KDAREF_GATE) && !A_log) return -1;
  if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || n_chains < 0) return -1;
  if (dtype != KDAREF_IO_F32 && dtype != KDAREF_IO_BF16) return -1;
  job_t jb;
  memset(&jb, 0, sizeof jb);
  jb.q = q; jb.k = k; jb.v = v; jb.dtype = dtype; jb.g = g; jb.beta = beta; jb.S0 = S0;
  jb.cu_seqlens = cu_seqlens; jb.B = B; jb.T = T; jb.H = H; jb.dk = dk; jb.dv = dv;
  jb.scale = scale; jb.delta_rule = delta_rule; jb.chains = chains; jb.n_chains = n_chains;
  jb.flags = flags; jb.A_log = A_log; jb.gate_bias = gate_bias;
  jb.out = out; jb.S_final = S_final;
  int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_chains > 0 ? n_chains : 1));
  int64_t acc = 0;
  for (int c = 0; c < n_chains; ++c) {
    const int n = chains[c] / H;
    if (chains[c] < 0 || n >= B) { free(off); return -1; }
    off[c] = acc;
    acc += cu_seqlens ? (int64_t)cu_seqlens[n + 1] - cu_seqlens[n] : (int64_t)T;
  }
  jb.out_offset = off;
  pthread_mutex_init(&jb.lock, NULL);
  if (threads < 1) threads = 1;
  if (threads > n_chains) threads = n_chains > 0 ? n_chains : 1;
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)threads);
  for (int i = 0; i < threads; ++i) pthread_create(&tid[i], NULL, worker, &jb);
  for (int i = 0; i < threads; ++i) pthread_join(tid[i], NULL);
  free(tid);
  pthread_mutex_destroy(&jb.lock);
  free(off);
  return 0;
}

/* kdaref_forward: kdaref_forward_ex without input transforms. */
int kdaref_forward(const void* q, const void* k, const void* v, int dtype,
                   const float* g, const float* beta, const double* S0,
                   const int32_t* cu_seqlens, int B, int T, int H, int dk, int dv,
                   double scale, int delta_rule, const int32_t* chains, int n_chains,
                   double* out, double* S_final, int threads) {
  return kdaref_forward_ex(q, k, v, dtype, g, beta, S0, cu_seqlens, B, T, H, dk, dv, scale,
                           delta_rule, 0, NULL, NULL, chains, n_chains, out, S_final, threads);
}
