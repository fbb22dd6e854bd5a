/*
 * flare_oracle.c -- plain fp64 CPU oracle for the dual-stream Gated DeltaNet
 * layer (clean causal stream + block-wise noisy stream), its reverse mode,
 * the serving block step and the dual-source causal ShortConv with its
 * reverse mode.
 *
 * THIS IS TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it.  It shares no code, header,
 * table or helper with the HIP library, and it does not know that library
 * exists.  Everything is a direct token-by-token transcription of the
 * definitions; there is no chunking, no blocking and no fusion.
 *
 * Sources (cited by key below):
 *   [KD2] "FLARE: Diffusion for Hybrid Language Model", papernotes.org notes,
 *         section "Key designs", item 2 (hybrid-attention state scheduling):
 *         the gated delta rule S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,
 *         the noisy block b starting from the clean boundary state S_{e(b-1)},
 *         and every position of the block reading the block-end state with
 *         the 1/sqrt(d_k) scale.
 *   [KD3] same page, "Key designs", item 3: ShortConv of width W whose taps
 *         that fall before the block start read the clean input and inside
 *         the block read the noisy input; cu_seqlens guard; documents packed
 *         with per-document reset and no cross-document gradient.
 *   [KD4] same page, "Key designs", item 4: denoising forwards never write the
 *         causal state pool; a causal replay writes the final state once the
 *         block is fixed.
 *   [FW]  same page, "Overall framework": the prompt is clean causal context
 *         only, the response is cut into consecutive blocks of B tokens.
 *   [TG]  Telegram post (quant_prune_distill/740), section "Method": the GDN
 *         state of a noisy block is the last clean block's state plus the
 *         noisy block's own contribution.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - S is d_k x d_v, outputs are o = s * S^T q with s = 1/sqrt(d_k) unless an
 *     explicit scale > 0 is given.
 *   - The decay a_t multiplies only (I - b_t k k^T) S_{t-1}, not the write term.
 *   - Noisy tokens carry their own a~, b~ gates.
 *   - Blocks are anchored at the first response token: boundaries are the
 *     clean-token counts P, P+B, P+2B, ... < n.  A boundary at 0 (P = 0) starts
 *     the block from the document's initial state.  A last block shorter than
 *     B reads the document end.
 *   - Noisy prompt rows are not read; their outputs and gradients are 0.
 *   - ShortConv taps follow a causal Conv1d: w[c, W-1] multiplies the current
 *     token; taps before the document start read 0.  Clean tokens of earlier
 *     response blocks are the clean history of a later block.
 *   - The optional q/k L2 normalisation divides by sqrt(sum x^2 + 1e-6).
 *
 * Parity pins for every function live in the CPU tests (closed forms,
 * invariants, brute-force matrix products, finite differences, a hand-worked
 * example); none of them re-types these loops.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define OR_FLAG_QK_L2NORM 1
#define OR_L2_EPS 1e-6

/* ------------------------------------------------------------------ */
/* small dense helpers (row-major, explicit loops)                      */
/* ------------------------------------------------------------------ */

/* One gated delta step on S (dk x dv), in place [KD2]:
 *   S <- a * (S - b k (k^T S)) + b k v^T.
 * If u_out is given it receives u = v - a S_prev^T k (used by reverse mode
 * checks only through the recomputation below). */
static void delta_step(double *S, int dk, int dv, const double *k,
                       const double *v, double a, double b, double *tmp) {
  /* tmp[j] = (k^T S)[j] */
  for (int j = 0; j < dv; ++j) tmp[j] = 0.0;
  for (int i = 0; i < dk; ++i) {
    const double ki = k[i];
    const double *row = S + (size_t)i * dv;
    for (int j = 0; j < dv; ++j) tmp[j] += ki * row[j];
  }
  for (int i = 0; i < dk; ++i) {
    const double ki = k[i];
    double *row = S + (size_t)i * dv;
    for (int j = 0; j < dv; ++j)
      row[j] = a * (row[j] - b * ki * tmp[j]) + b * ki * v[j];
  }
}

/* out[j] = s * sum_i S[i][j] q[i]   (o = s S^T q)  [KD2] */
static void read_state(const double *S, int dk, int dv, const double *q,
                       double s, double *out) {
  for (int j = 0; j < dv; ++j) out[j] = 0.0;
  for (int i = 0; i < dk; ++i) {
    const double qi = q[i];
    const double *row = S + (size_t)i * dv;
    for (int j = 0; j < dv; ++j) out[j] += qi * row[j];
  }
  for (int j = 0; j < dv; ++j) out[j] *= s;
}

static void l2norm_copy(const double *x, int d, double *y) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += x[i] * x[i];
  const double r = 1.0 / sqrt(ss + OR_L2_EPS);
  for (int i = 0; i < d; ++i) y[i] = x[i] * r;
}

/* dx = (dy - y (y.dy)) / sqrt(|x|^2 + eps), the derivative of l2norm_copy. */
static void l2norm_back(const double *x, int d, const double *dy, double *dx) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += x[i] * x[i];
  const double r = sqrt(ss + OR_L2_EPS);
  double ydy = 0.0;
  for (int i = 0; i < d; ++i) ydy += (x[i] / r) * dy[i];
  for (int i = 0; i < d; ++i) dx[i] = (dy[i] - (x[i] / r) * ydy) / r;
}

static double resolve_scale(double scale, int dk) {
  return scale > 0.0 ? scale : 1.0 / sqrt((double)dk);
}

/* ------------------------------------------------------------------ */
/* thread pool over independent units                                  */
/* ------------------------------------------------------------------ */

typedef void (*unit_fn)(void *ctx, int unit, void *scratch);

typedef struct {
  unit_fn fn;
  void *ctx;
  int n_units;
  int next;
  size_t scratch_bytes;
  pthread_mutex_t mu;
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *p = (pool_t *)arg;
  void *scratch = malloc(p->scratch_bytes ? p->scratch_bytes : 1);
  for (;;) {
    pthread_mutex_lock(&p->mu);
    int u = p->next++;
    pthread_mutex_unlock(&p->mu);
    if (u >= p->n_units) break;
    p->fn(p->ctx, u, scratch);
  }
  free(scratch);
  return NULL;
}

int oracle_default_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

static void run_units(unit_fn fn, void *ctx, int n_units, size_t scratch_bytes,
                      int nthreads) {
  if (nthreads <= 0) nthreads = oracle_default_threads();
  if (nthreads > n_units) nthreads = n_units > 0 ? n_units : 1;
  pool_t p;
  p.fn = fn;
  p.ctx = ctx;
  p.n_units = n_units;
  p.next = 0;
  p.scratch_bytes = scratch_bytes;
  pthread_mutex_init(&p.mu, NULL);
  if (nthreads <= 1) {
    pool_worker(&p);
  } else {
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, pool_worker, &p);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&p.mu);
}

/* ------------------------------------------------------------------ */
/* dual-stream forward [KD2][FW][KD3][TG]                              */
/* ------------------------------------------------------------------ */

typedef struct {
  int num_docs, H, dk, dv, B, flags;
  double s;
  const int32_t *cu, *plen;
  const double *q, *k, *v, *a, *b;
  const double *qn, *kn, *vn, *an, *bn;
  const double *h0;
  double *o, *on, *h_final;
} fwd_ctx;

/* Fetch a q/k-like row of token t (global), head h, optionally L2-normalised. */
static const double *row_of(const double *x, int t, int h, int H, int d,
                            int norm, double *buf) {
  const double *r = x + ((size_t)t * H + h) * d;
  if (!norm) return r;
  l2norm_copy(r, d, buf);
  return buf;
}

static void fwd_unit(void *vctx, int unit, void *scratch) {
  fwd_ctx *c = (fwd_ctx *)vctx;
  const int doc = unit / c->H, h = unit % c->H;
  const int H = c->H, dk = c->dk, dv = c->dv, B = c->B;
  const int start = c->cu[doc], n = c->cu[doc + 1] - c->cu[doc];
  const int P = c->plen[doc];
  const int norm = (c->flags & OR_FLAG_QK_L2NORM) != 0;
  double *S = (double *)scratch;              /* dk*dv clean state   */
  double *Sn = S + (size_t)dk * dv;           /* dk*dv noisy copy    */
  double *tmp = Sn + (size_t)dk * dv;         /* dv                  */
  double *bq = tmp + dv, *bk = bq + dk;       /* normalised rows     */
  const size_t SS = (size_t)dk * dv;

  if (c->h0) memcpy(S, c->h0 + ((size_t)doc * H + h) * SS, SS * sizeof(double));
  else memset(S, 0, SS * sizeof(double));

  /* noisy prompt rows are zero by definition */
  for (int t = 0; t < P && t < n; ++t)
    memset(c->on + ((size_t)(start + t) * H + h) * dv, 0, dv * sizeof(double));

  for (int t = 0; t <= n; ++t) {
    /* t = number of clean tokens already absorbed into S */
    if (t > 0) {
      const int g = start + t - 1;
      const double *kt = row_of(c->k, g, h, H, dk, norm, bk);
      delta_step(S, dk, dv, kt, c->v + ((size_t)g * H + h) * dv,
                 c->a[(size_t)g * H + h], c->b[(size_t)g * H + h], tmp);
      const double *qt = row_of(c->q, g, h, H, dk, norm, bq);
      read_state(S, dk, dv, qt, c->s, c->o + ((size_t)g * H + h) * dv);
    }
    if (t >= P && t < n && ((t - P) % B) == 0) {
      /* noisy block covering tokens t .. e-1 starts from the clean state S_t */
      const int e = (t + B < n) ? t + B : n;
      memcpy(Sn, S, SS * sizeof(double));
      for (int l = t; l < e; ++l) {
        const int g = start + l;
        const double *kl = row_of(c->kn, g, h, H, dk, norm, bk);
        delta_step(Sn, dk, dv, kl, c->vn + ((size_t)g * H + h) * dv,
                   c->an[(size_t)g * H + h], c->bn[(size_t)g * H + h], tmp);
      }
      /* every position of the block reads the block-end state */
      for (int l = t; l < e; ++l) {
        const int g = start + l;
        const double *ql = row_of(c->qn, g, h, H, dk, norm, bq);
        read_state(Sn, dk, dv, ql, c->s, c->on + ((size_t)g * H + h) * dv);
      }
    }
  }
  if (c->h_final) memcpy(c->h_final + ((size_t)doc * H + h) * SS, S, SS * sizeof(double));
}

int oracle_gdn_dual_fwd(int num_docs, const int32_t *cu_seqlens,
                        const int32_t *prompt_lens, int H, int dk, int dv,
                        int B, double scale, int flags, const double *q,
                        const double *k, const double *v, const double *a,
                        const double *b, const double *qn, const double *kn,
                        const double *vn, const double *an, const double *bn,
                        const double *h0, double *o, double *on,
                        double *h_final, int nthreads) {
  if (num_docs < 0 || H <= 0 || dk <= 0 || dv <= 0 || B <= 0) return 2;
  for (int i = 0; i < num_docs; ++i) {
    const int n = cu_seqlens[i + 1] - cu_seqlens[i];
    if (n < 0 || prompt_lens[i] < 0 || prompt_lens[i] > n) return 2;
  }
  fwd_ctx c = {num_docs, H, dk, dv, B, flags, resolve_scale(scale, dk),
               cu_seqlens, prompt_lens, q, k, v, a, b, qn, kn, vn, an, bn,
               h0, o, on, h_final};
  const size_t scratch = (2 * (size_t)dk * dv + dv + 2 * (size_t)dk) * sizeof(double);
  run_units(fwd_unit, &c, num_docs * H, scratch, nthreads);
  return 0;
}

/* ------------------------------------------------------------------ */
/* reverse mode of the dual-stream forward [KD2][KD3]                  */
/* ------------------------------------------------------------------ */
/*
 * For one step S = a S' + b k u^T with u = v - a S'^T k and upstream
 * adjoint G = dL/dS:
 *   dv = b G^T k,   db = k^T G u,   da = <G,S'> - b k^T G S'^T k,
 *   dk = b G u - a b S' (G^T k),    dL/dS' = a (G - b k (k^T G)).
 * A read o = s S^T q adds s q do^T to dL/dS and gives dq = s S do.
 * The adjoint reaching the start of a noisy block is added to the clean
 * adjoint at that block's boundary ("block gradients injected into the causal
 * main chain", [KD2]); the adjoint is reset per document [KD3].
 */

typedef struct {
  int num_docs, H, dk, dv, B, flags, ck;
  double s;
  const int32_t *cu, *plen;
  const double *q, *k, *v, *a, *b;
  const double *qn, *kn, *vn, *an, *bn;
  const double *h0;
  const double *dout, *dout_n, *dh_final;
  double *dq, *dk_, *dv_, *da, *db;
  double *dqn, *dkn, *dvn, *dan, *dbn, *dh0;
} bwd_ctx;

/* backward of one step; G is updated in place to dL/dS'.  k is the (possibly
 * normalised) key; dk_out receives the gradient w.r.t. that key. */
static void step_back(double *G, const double *Sp, int dk, int dv,
                      const double *k, const double *v, double a, double b,
                      double *dk_out, double *dv_out, double *da_out,
                      double *db_out, double *w1, double *w2) {
  /* w1 = S'^T k (dv), u = v - a w1 (stored in w1 afterwards) */
  for (int j = 0; j < dv; ++j) w1[j] = 0.0;
  for (int i = 0; i < dk; ++i) {
    const double *row = Sp + (size_t)i * dv;
    for (int j = 0; j < dv; ++j) w1[j] += k[i] * row[j];
  }
  /* w2 = G^T k (dv) */
  for (int j = 0; j < dv; ++j) w2[j] = 0.0;
  for (int i = 0; i < dk; ++i) {
    const double *row = G + (size_t)i * dv;
    for (int j = 0; j < dv; ++j) w2[j] += k[i] * row[j];
  }
  /* da = <G,S'> - b (G^T k).(S'^T k) */
  double gs = 0.0, w12 = 0.0;
  for (size_t e = 0; e < (size_t)dk * dv; ++e) gs += G[e] * Sp[e];
  for (int j = 0; j < dv; ++j) w12 += w2[j] * w1[j];
  *da_out = gs - b * w12;
  /* u = v - a w1 */
  double dbv = 0.0;
  for (int j = 0; j < dv; ++j) {
    w1[j] = v[j] - a * w1[j];
    dbv += w2[j] * w1[j];
  }
  *db_out = dbv; /* k^T G u = (G^T k).u */
  for (int j = 0; j < dv; ++j) dv_out[j] = b * w2[j];
  /* dk = b G u - a b S' w2 */
  for (int i = 0; i < dk; ++i) {
    const double *gr = G + (size_t)i * dv;
    const double *sr = Sp + (size_t)i * dv;
    double x = 0.0, y = 0.0;
    for (int j = 0; j < dv; ++j) {
      x += gr[j] * w1[j];
      y += sr[j] * w2[j];
    }
    dk_out[i] = b * x - a * b * y;
  }
  /* G <- a (G - b k w2^T) */
  for (int i = 0; i < dk; ++i) {
    double *gr = G + (size_t)i * dv;
    for (int j = 0; j < dv; ++j) gr[j] = a * (gr[j] - b * k[i] * w2[j]);
  }
}

/* add s x dy^T into G (read adjoint), and write dx = s S dy */
static void read_back(double *G, const double *S, int dk, int dv,
                      const double *x, const double *dy, double s,
                      double *dx_out) {
  for (int i = 0; i < dk; ++i) {
    double *gr = G + (size_t)i * dv;
    const double *sr = S + (size_t)i * dv;
    double acc = 0.0;
    for (int j = 0; j < dv; ++j) {
      gr[j] += s * x[i] * dy[j];
      acc += sr[j] * dy[j];
    }
    dx_out[i] = s * acc;
  }
}

typedef struct {
  double *S, *Sn_all, *G, *Gn, *ck_states, *w1, *w2, *rq, *rk, *drq, *drk;
} bwd_scratch;

static void bwd_scratch_bind(bwd_scratch *w, void *raw, int dk, int dv, int B,
                             int ck) {
  const size_t SS = (size_t)dk * dv;
  double *p = (double *)raw;
  w->S = p; p += SS;
  w->G = p; p += SS;
  w->Gn = p; p += SS;
  w->Sn_all = p; p += SS * (size_t)(B + 1);
  w->ck_states = p; p += SS * (size_t)(ck + 1);
  w->w1 = p; p += dv > dk ? dv : dk;
  w->w2 = p; p += dv > dk ? dv : dk;
  w->rq = p; p += dk;
  w->rk = p; p += dk;
  w->drq = p; p += dk;
  w->drk = p; p += dk;
}

static size_t bwd_scratch_bytes(int dk, int dv, int B, int ck) {
  const size_t SS = (size_t)dk * dv;
  const size_t m = (size_t)(dv > dk ? dv : dk);
  return (SS * (3 + (size_t)(B + 1) + (size_t)(ck + 1)) + 2 * m + 4 * (size_t)dk) *
         sizeof(double);
}

/* Backward of the noisy block that starts from clean state Sp (boundary at
 * clean count t, tokens t..e-1).  Accumulates the block-start adjoint into
 * Gclean and writes the noisy-token gradients. */
static void noisy_block_back(bwd_ctx *c, bwd_scratch *w, int doc, int h, int t,
                             int e, const double *Sp, double *Gclean) {
  const int H = c->H, dk = c->dk, dv = c->dv;
  const int start = c->cu[doc];
  const int norm = (c->flags & OR_FLAG_QK_L2NORM) != 0;
  const size_t SS = (size_t)dk * dv;
  const int nb = e - t;
  /* recompute noisy states Sn_all[0..nb] */
  memcpy(w->Sn_all, Sp, SS * sizeof(double));
  for (int l = 0; l < nb; ++l) {
    const int g = start + t + l;
    double *Sl = w->Sn_all + SS * (size_t)(l + 1);
    memcpy(Sl, w->Sn_all + SS * (size_t)l, SS * sizeof(double));
    const double *kl = row_of(c->kn, g, h, H, dk, norm, w->rk);
    delta_step(Sl, dk, dv, kl, c->vn + ((size_t)g * H + h) * dv,
               c->an[(size_t)g * H + h], c->bn[(size_t)g * H + h], w->w1);
  }
  const double *Se = w->Sn_all + SS * (size_t)nb;
  /* block-end reads: every position reads Se */
  memset(w->Gn, 0, SS * sizeof(double));
  for (int l = 0; l < nb; ++l) {
    const int g = start + t + l;
    const size_t r = (size_t)g * H + h;
    const double *ql = row_of(c->qn, g, h, H, dk, norm, w->rq);
    read_back(w->Gn, Se, dk, dv, ql, c->dout_n + r * dv, c->s, w->drq);
    if (norm) l2norm_back(c->qn + r * dk, dk, w->drq, c->dqn + r * dk);
    else memcpy(c->dqn + r * dk, w->drq, dk * sizeof(double));
  }
  for (int l = nb - 1; l >= 0; --l) {
    const int g = start + t + l;
    const size_t r = (size_t)g * H + h;
    const double *kl = row_of(c->kn, g, h, H, dk, norm, w->rk);
    step_back(w->Gn, w->Sn_all + SS * (size_t)l, dk, dv, kl,
              c->vn + r * dv, c->an[r], c->bn[r], w->drk, c->dvn + r * dv,
              &c->dan[r], &c->dbn[r], w->w1, w->w2);
    if (norm) l2norm_back(c->kn + r * dk, dk, w->drk, c->dkn + r * dk);
    else memcpy(c->dkn + r * dk, w->drk, dk * sizeof(double));
  }
  for (size_t x = 0; x < SS; ++x) Gclean[x] += w->Gn[x];
}

static void bwd_unit(void *vctx, int unit, void *scratch) {
  bwd_ctx *c = (bwd_ctx *)vctx;
  const int doc = unit / c->H, h = unit % c->H;
  const int H = c->H, dk = c->dk, dv = c->dv, B = c->B, CK = c->ck;
  const int start = c->cu[doc], n = c->cu[doc + 1] - c->cu[doc];
  const int P = c->plen[doc];
  const int norm = (c->flags & OR_FLAG_QK_L2NORM) != 0;
  const size_t SS = (size_t)dk * dv;
  bwd_scratch w;
  bwd_scratch_bind(&w, scratch, dk, dv, B, CK);

  /* zero noisy prompt-row gradients */
  for (int t = 0; t < P && t < n; ++t) {
    const size_t r = (size_t)(start + t) * H + h;
    memset(c->dqn + r * dk, 0, dk * sizeof(double));
    memset(c->dkn + r * dk, 0, dk * sizeof(double));
    memset(c->dvn + r * dv, 0, dv * sizeof(double));
    c->dan[r] = 0.0;
    c->dbn[r] = 0.0;
  }

  /* forward pass keeping a state every CK steps (fp64, oracle-internal) */
  const int n_seg = n / CK + 1;
  double *seg_start = (double *)malloc(SS * (size_t)n_seg * sizeof(double));
  if (c->h0) memcpy(w.S, c->h0 + ((size_t)doc * H + h) * SS, SS * sizeof(double));
  else memset(w.S, 0, SS * sizeof(double));
  for (int t = 0; t < n; ++t) {
    if (t % CK == 0) memcpy(seg_start + SS * (size_t)(t / CK), w.S, SS * sizeof(double));
    const int g = start + t;
    const double *kt = row_of(c->k, g, h, H, dk, norm, w.rk);
    delta_step(w.S, dk, dv, kt, c->v + ((size_t)g * H + h) * dv,
               c->a[(size_t)g * H + h], c->b[(size_t)g * H + h], w.w1);
  }
  if (n % CK == 0) memcpy(seg_start + SS * (size_t)(n / CK), w.S, SS * sizeof(double));

  /* reverse sweep */
  if (c->dh_final) memcpy(w.G, c->dh_final + ((size_t)doc * H + h) * SS, SS * sizeof(double));
  else memset(w.G, 0, SS * sizeof(double));

  int cur_seg = -1;
  for (int t = n; t >= 1; --t) {
    /* need S_t and S_{t-1}: states of segment (t-1)/CK */
    const int seg = (t - 1) / CK;
    if (seg != cur_seg) {
      /* rebuild ck_states[0..len] = S_{seg*CK + j} */
      const int t0 = seg * CK;
      const int len = (t0 + CK <= n) ? CK : n - t0;
      memcpy(w.ck_states, seg_start + SS * (size_t)seg, SS * sizeof(double));
      for (int j = 0; j < len; ++j) {
        double *Sj = w.ck_states + SS * (size_t)(j + 1);
        memcpy(Sj, w.ck_states + SS * (size_t)j, SS * sizeof(double));
        const int g = start + t0 + j;
        const double *kt = row_of(c->k, g, h, H, dk, norm, w.rk);
        delta_step(Sj, dk, dv, kt, c->v + ((size_t)g * H + h) * dv,
                   c->a[(size_t)g * H + h], c->b[(size_t)g * H + h], w.w1);
      }
      cur_seg = seg;
    }
    const int t0 = seg * CK;
    const double *St = w.ck_states + SS * (size_t)(t - t0);
    const double *Sp = w.ck_states + SS * (size_t)(t - 1 - t0);
    const int g = start + t - 1;
    const size_t r = (size_t)g * H + h;
    /* o_t reads S_t */
    const double *qt = row_of(c->q, g, h, H, dk, norm, w.rq);
    read_back(w.G, St, dk, dv, qt, c->dout + r * dv, c->s, w.drq);
    if (norm) l2norm_back(c->q + r * dk, dk, w.drq, c->dq + r * dk);
    else memcpy(c->dq + r * dk, w.drq, dk * sizeof(double));
    /* the noisy block whose boundary is t reads S_t as its start */
    if (t >= P && t < n && ((t - P) % B) == 0) {
      const int e = (t + B < n) ? t + B : n;
      noisy_block_back(c, &w, doc, h, t, e, St, w.G);
    }
    /* step t */
    const double *kt = row_of(c->k, g, h, H, dk, norm, w.rk);
    step_back(w.G, Sp, dk, dv, kt, c->v + r * dv, c->a[r], c->b[r], w.drk,
              c->dv_ + r * dv, &c->da[r], &c->db[r], w.w1, w.w2);
    if (norm) l2norm_back(c->k + r * dk, dk, w.drk, c->dk_ + r * dk);
    else memcpy(c->dk_ + r * dk, w.drk, dk * sizeof(double));
  }
  if (P == 0 && n > 0) {
    /* first block starts from the document's initial state */
    const double *S0 = seg_start; /* S_0 */
    const int e = (B < n) ? B : n;
    noisy_block_back(c, &w, doc, h, 0, e, S0, w.G);
  }
  if (c->dh0) memcpy(c->dh0 + ((size_t)doc * H + h) * SS, w.G, SS * sizeof(double));
  free(seg_start);
}

int oracle_gdn_dual_bwd(int num_docs, const int32_t *cu_seqlens,
                        const int32_t *prompt_lens, int H, int dk, int dv,
                        int B, double scale, int flags, const double *q,
                        const double *k, const double *v, const double *a,
                        const double *b, const double *qn, const double *kn,
                        const double *vn, const double *an, const double *bn,
                        const double *h0, const double *dout,
                        const double *dout_n, const double *dh_final,
                        double *dq, double *dk_, double *dv_, double *da,
                        double *db, double *dqn, double *dkn, double *dvn,
                        double *dan, double *dbn, double *dh0, int nthreads) {
  if (num_docs < 0 || H <= 0 || dk <= 0 || dv <= 0 || B <= 0) return 2;
  for (int i = 0; i < num_docs; ++i) {
    const int n = cu_seqlens[i + 1] - cu_seqlens[i];
    if (n < 0 || prompt_lens[i] < 0 || prompt_lens[i] > n) return 2;
  }
  const int CK = 64;
  bwd_ctx c = {num_docs, H, dk, dv, B, flags, CK, resolve_scale(scale, dk),
               cu_seqlens, prompt_lens, q, k, v, a, b, qn, kn, vn, an, bn, h0,
               dout, dout_n, dh_final, dq, dk_, dv_, da, db, dqn, dkn, dvn,
               dan, dbn, dh0};
  run_units(bwd_unit, &c, num_docs * H, bwd_scratch_bytes(dk, dv, B, CK), nthreads);
  return 0;
}

/* ------------------------------------------------------------------ */
/* serving block step [KD4]                                            */
/* ------------------------------------------------------------------ */

typedef struct {
  int num_req, H, dk, dv, B, mode;
  double s;
  const int32_t *slot;
  double *pool;
  const double *q, *k, *v, *a, *b;
  double *o;
  double *cand; /* VERIFY: [num_req, B, H, dk, dv] states after each token */
} step_ctx;

/* mode 0 (EVAL): apply the B noisy updates to a private copy of the pooled
 *   state; every position reads the block-end state; the pool is untouched.
 * mode 1 (COMMIT): replay the B committed tokens causally on the pooled
 *   state with a per-token read after each update, then write it back. */
static void step_unit(void *vctx, int unit, void *scratch) {
  step_ctx *c = (step_ctx *)vctx;
  const int r = unit / c->H, h = unit % c->H;
  const int H = c->H, dk = c->dk, dv = c->dv, B = c->B;
  const size_t SS = (size_t)dk * dv;
  double *S = (double *)scratch;
  double *tmp = S + SS;
  double *P = c->pool + ((size_t)c->slot[r] * H + h) * SS;
  memcpy(S, P, SS * sizeof(double));
  for (int l = 0; l < B; ++l) {
    const size_t row = ((size_t)r * B + l) * H + h;
    delta_step(S, dk, dv, c->k + row * dk, c->v + row * dv, c->a[row], c->b[row], tmp);
    if (c->mode >= 1 && c->o) read_state(S, dk, dv, c->q + row * dk, c->s, c->o + row * dv);
    if (c->mode == 2) memcpy(c->cand + row * SS, S, SS * sizeof(double));
  }
  if (c->mode == 2) return; /* VERIFY leaves the pool as it was */
  if (c->mode == 0) {
    for (int l = 0; l < B; ++l) {
      const size_t row = ((size_t)r * B + l) * H + h;
      read_state(S, dk, dv, c->q + row * dk, c->s, c->o + row * dv);
    }
  } else {
    memcpy(P, S, SS * sizeof(double));
  }
}

int oracle_block_step(int num_req, const int32_t *slot_idx, double *pool,
                      int num_slots, int H, int dk, int dv, int B,
                      double scale, const double *q, const double *k,
                      const double *v, const double *a, const double *b,
                      double *o, int mode, int nthreads) {
  if (num_req < 0 || H <= 0 || dk <= 0 || dv <= 0 || B <= 0) return 2;
  if (mode != 0 && mode != 1) return 2;
  for (int r = 0; r < num_req; ++r) {
    if (slot_idx[r] < 0 || slot_idx[r] >= num_slots) return 2;
    for (int j = 0; j < r; ++j)
      if (slot_idx[j] == slot_idx[r]) return 2;
  }
  step_ctx c = {num_req, H, dk, dv, B, mode, resolve_scale(scale, dk),
                slot_idx, pool, q, k, v, a, b, o, NULL};
  run_units(step_unit, &c, num_req * H, ((size_t)dk * dv + dv) * sizeof(double), nthreads);
  return 0;
}

/* AR-Trust verify [KD4]: the clean causal pass over K drafted tokens from the
 * pool state, as COMMIT (per-token outputs o_t = s S_t^T q_t), except that the
 * state after every token goes to cand[r][t] and the pool is not written. */
int oracle_gdn_verify(int num_req, const int32_t *slot_idx, double *pool,
                      int num_slots, int H, int dk, int dv, int K,
                      double scale, const double *q, const double *k,
                      const double *v, const double *a, const double *b,
                      double *o, double *cand, int nthreads) {
  if (num_req < 0 || H <= 0 || dk <= 0 || dv <= 0 || K <= 0 || !cand) return 2;
  for (int r = 0; r < num_req; ++r) {
    if (slot_idx[r] < 0 || slot_idx[r] >= num_slots) return 2;
    for (int j = 0; j < r; ++j)
      if (slot_idx[j] == slot_idx[r]) return 2;
  }
  step_ctx c = {num_req, H, dk, dv, K, 2, resolve_scale(scale, dk),
                slot_idx, pool, q, k, v, a, b, o, cand};
  run_units(step_unit, &c, num_req * H, ((size_t)dk * dv + dv) * sizeof(double), nthreads);
  return 0;
}

/* ------------------------------------------------------------------ */
/* dual-source causal ShortConv [KD3]                                  */
/* ------------------------------------------------------------------ */

typedef struct {
  int num_docs, B, C, W, activation;
  const int32_t *cu, *plen;
  const double *x, *xn, *w, *bias;
  double *y, *yn;
} conv_ctx;

static double act(double z, int activation) {
  return activation == 1 ? z / (1.0 + exp(-z)) : z;
}

/* y^c[t] = sum_j w[j] x^c[t-(W-1)+j]; a noisy tap at position m reads x^c[m]
 * when m lies before the start of t's block and x^n[m] inside the block. */
static void conv_unit(void *vctx, int doc, void *scratch) {
  (void)scratch;
  conv_ctx *c = (conv_ctx *)vctx;
  const int C = c->C, W = c->W, B = c->B;
  const int start = c->cu[doc], n = c->cu[doc + 1] - c->cu[doc];
  const int P = c->plen[doc];
  for (int t = 0; t < n; ++t) {
    const int blk = (t >= P) ? P + ((t - P) / B) * B : -1;
    for (int ch = 0; ch < C; ++ch) {
      double acc_c = c->bias ? c->bias[ch] : 0.0;
      double acc_n = acc_c;
      for (int j = 0; j < W; ++j) {
        const int m = t - (W - 1) + j;
        if (m < 0) continue;
        const double wj = c->w[(size_t)ch * W + j];
        const double xc = c->x[(size_t)(start + m) * C + ch];
        acc_c += wj * xc;
        if (blk >= 0) acc_n += wj * (m < blk ? xc : c->xn[(size_t)(start + m) * C + ch]);
      }
      c->y[(size_t)(start + t) * C + ch] = act(acc_c, c->activation);
      c->yn[(size_t)(start + t) * C + ch] = blk >= 0 ? act(acc_n, c->activation) : 0.0;
    }
  }
}

/* Reverse mode of the ShortConv above: with z the pre-activation sums and
 * g = dy * act'(z) (g~ = dy~ * act'(z~) on response rows, 0 on prompt rows),
 * every tap that read input element m passes w[j] * g to that element's
 * gradient -- the clean input's, or the noisy input's when the noisy tap read
 * x~ -- and w[j] receives g times the value the tap read; the bias receives g.
 * One unit per channel, so each unit owns its dw row, its dbias entry and its
 * column of dx, dx~. */
typedef struct {
  int num_docs, B, C, W, activation;
  const int32_t *cu, *plen;
  const double *x, *xn, *w, *bias, *dy, *dyn;
  double *dx, *dxn, *dw, *db;
} convb_ctx;

static double act_grad(double z, int activation) {
  if (activation != 1) return 1.0;
  const double sg = 1.0 / (1.0 + exp(-z));
  return sg * (1.0 + z * (1.0 - sg));
}

static void convb_unit(void *vctx, int ch, void *scratch) {
  (void)scratch;
  convb_ctx *c = (convb_ctx *)vctx;
  const int C = c->C, W = c->W, B = c->B;
  const double *wr = c->w + (size_t)ch * W;
  double *dwr = c->dw + (size_t)ch * W;
  for (int j = 0; j < W; ++j) dwr[j] = 0.0;
  double db = 0.0;
  for (int doc = 0; doc < c->num_docs; ++doc) {
    const int start = c->cu[doc], n = c->cu[doc + 1] - c->cu[doc];
    const int P = c->plen[doc];
    for (int t = 0; t < n; ++t) {
      c->dx[(size_t)(start + t) * C + ch] = 0.0;
      c->dxn[(size_t)(start + t) * C + ch] = 0.0;
    }
    for (int t = 0; t < n; ++t) {
      const int blk = (t >= P) ? P + ((t - P) / B) * B : -1;
      /* the forward sums again, for the activation's derivative */
      double zc = c->bias ? c->bias[ch] : 0.0, zn = zc;
      for (int j = 0; j < W; ++j) {
        const int m = t - (W - 1) + j;
        if (m < 0) continue;
        const double xc = c->x[(size_t)(start + m) * C + ch];
        zc += wr[j] * xc;
        if (blk >= 0) zn += wr[j] * (m < blk ? xc : c->xn[(size_t)(start + m) * C + ch]);
      }
      const double gc = c->dy[(size_t)(start + t) * C + ch] * act_grad(zc, c->activation);
      const double gn = blk >= 0 ? c->dyn[(size_t)(start + t) * C + ch] * act_grad(zn, c->activation) : 0.0;
      db += gc + gn;
      for (int j = 0; j < W; ++j) {
        const int m = t - (W - 1) + j;
        if (m < 0) continue;
        const size_t at = (size_t)(start + m) * C + ch;
        c->dx[at] += wr[j] * gc;
        dwr[j] += gc * c->x[at];
        if (blk >= 0) {
          if (m < blk) {
            c->dx[at] += wr[j] * gn;
            dwr[j] += gn * c->x[at];
          } else {
            c->dxn[at] += wr[j] * gn;
            dwr[j] += gn * c->xn[at];
          }
        }
      }
    }
  }
  if (c->db) c->db[ch] = db;
}

int oracle_shortconv_dual_bwd(int num_docs, const int32_t *cu_seqlens,
                              const int32_t *prompt_lens, int B, int channels,
                              int width, const double *x, const double *xn,
                              const double *weight, const double *bias,
                              int activation, const double *dy, const double *dyn,
                              double *dx, double *dxn, double *dweight,
                              double *dbias, int nthreads) {
  if (num_docs < 0 || B <= 0 || channels <= 0 || width <= 0) return 2;
  for (int i = 0; i < num_docs; ++i) {
    const int n = cu_seqlens[i + 1] - cu_seqlens[i];
    if (n < 0 || prompt_lens[i] < 0 || prompt_lens[i] > n) return 2;
  }
  convb_ctx c = {num_docs, B, channels, width, activation, cu_seqlens, prompt_lens,
                 x, xn, weight, bias, dy, dyn, dx, dxn, dweight, dbias};
  run_units(convb_unit, &c, channels, 0, nthreads);
  return 0;
}

int oracle_shortconv_dual(int num_docs, const int32_t *cu_seqlens,
                          const int32_t *prompt_lens, int B, int channels,
                          int width, const double *x, const double *xn,
                          const double *weight, const double *bias,
                          int activation, double *y, double *yn,
                          int nthreads) {
  if (num_docs < 0 || B <= 0 || channels <= 0 || width <= 0) return 2;
  for (int i = 0; i < num_docs; ++i) {
    const int n = cu_seqlens[i + 1] - cu_seqlens[i];
    if (n < 0 || prompt_lens[i] < 0 || prompt_lens[i] > n) return 2;
  }
  conv_ctx c = {num_docs, B, channels, width, activation, cu_seqlens,
                prompt_lens, x, xn, weight, bias, y, yn};
  run_units(conv_unit, &c, num_docs, 0, nthreads);
  return 0;
}
