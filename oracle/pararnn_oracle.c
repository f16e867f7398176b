/*
 * pararnn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU statement of what the ParaRNN hot path computes.
 * It exists so that the GPU library can be checked against something that a
 * reader can verify by eye.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header or table with the GPU library.
 *
 * Sources (the pages are cited by title and section):
 *  - pararnn-torch README (PyPI page), section "Method": the whole hidden
 *    trajectory H is the unknown of F(H)_t = h_t - f(h_{t-1}, x_t) = 0, solved
 *    with Newton updates whose linear solves are associative scans over time.
 *  - same page, "Method": the backward pass follows the paper's adjoint
 *    equation (a reverse linear recurrence with transposed Jacobians).
 *  - ParaRNN abstract (HF paper list): Newton iterations combined with
 *    parallel reductions; it trains LSTM- and GRU-like cells this way.
 *  - The diagonal GRU cell equations are the benchmark statement that comes
 *    with this code base; the LSTM is the textbook cell without peepholes
 *    whose recurrent weights are diagonal and act on h (a reading: the pages
 *    print no LSTM equations).
 *
 * Everything is sequential in time and in fp64; std C math (exp, tanh) only.
 * Threads split the B*D independent channels; each channel walks T serially.
 *
 * Parity pins: see tests/test_oracle_*.py.  Every function below is pinned by
 * a closed form, a brute-force sum, a library routine (torch GRUCell /
 * LSTMCell, numpy.linalg.solve, autograd) or a finite-difference check.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_LINEAR = 0, OR_GRU = 1, OR_LSTM = 2, OR_SLSTM = 3, OR_HGRU = 4 };
/* largest state size and gate count of the cells below */
enum { OR_SMAX = 4, OR_GMAX = 4 };
enum { OR_OK = 0, OR_EINVAL = -1, OR_ENOMEM = -2, OR_DIVERGED = -5 };

/* ------------------------------------------------------------------------ */
/* input decoding                                                           */
/* ------------------------------------------------------------------------ */

/* A bf16 value is the upper half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t v) {
  uint32_t u = (uint32_t)v << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load_in(const void* p, int dtype, int64_t i) {
  if (dtype == OR_BF16) return bf16_bits_to_double(((const uint16_t*)p)[i]);
  return (double)((const float*)p)[i];
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static int state_size(int cell) { return cell == OR_SLSTM ? 4 : (cell == OR_LSTM ? 2 : 1); }
static int gate_count(int cell) {
  return (cell == OR_LSTM || cell == OR_SLSTM) ? 4 : ((cell == OR_GRU || cell == OR_HGRU) ? 3 : 2);
}

/* log(sigmoid(x)) without overflow for either sign of x */
static double log_sigmoid(double x) { return x >= 0.0 ? -log1p(exp(-x)) : x - log1p(exp(x)); }

/* ------------------------------------------------------------------------ */
/* one cell step                                                            */
/* ------------------------------------------------------------------------ */

/*
 * or_cell_step: s_next = f(s, x) for one channel, with
 *   J[S*S]     = d s_next / d s        (row-major: J[i*S+j] = d s_next_i / d s_j)
 *   dfdu[S*G]  = d s_next / d u_g      (dfdu[i*G+g]), u_g the full gate
 *                pre-activation  u_g = U_g + w_g * (input of w_g) + bias_g
 *   wcoef[G]   = the factor that multiplies w_g inside u_g
 * Any of J, dfdu, wcoef may be NULL.
 *
 * GRU (state h; gates z, r, c; benchmark statement of the diagonal GRU):
 *   z = sig(U_z + a_z h + b_z),  r = sig(U_r + a_r h + b_r)
 *   c = tanh(U_c + a_c (r h) + b_c),  h' = (1 - z) h + z c
 * LSTM (state (c, h); gates i, f, o, g; textbook cell, diagonal w on h):
 *   i,f,o = sig(U + w h + b),  g = tanh(U_g + w_g h + b_g)
 *   c' = f c + i g,  h' = o tanh(c')
 * sLSTM, diagonal recurrence (state (c, n, m, h); gates z, i, f, o): the
 * published sLSTM (xLSTM, Beck et al. 2024) with exponential input gate,
 * sigmoid forget gate and its log-domain stabiliser m (a reading: the pages
 * name the cell, ParaSLSTM with mix="diag", but print no equations):
 *   u_g = U_g + w_g h + b_g,  z = tanh(u_z),  o = sig(u_o),  lf = log sig(u_f)
 *   m' = max(lf + m, u_i),  i' = exp(u_i - m'),  f' = exp(lf + m - m')
 *   c' = f' c + i' z,  n' = f' n + i',  h' = o c' / n'
 * At a tie of the max the forget branch is taken; its derivative is the
 * branch's (the max is piecewise linear).
 * LINEAR (state h; "gates" a, b are the coefficients themselves):
 *   h' = a h + b
 * u[] for LINEAR holds (a_t, b_t); w and bias are ignored.
 */
int or_cell_step(int cell, const double* u_in, const double* w,
                 const double* bias, const double* s, double* s_next,
                 double* J, double* dfdu, double* wcoef) {
  if (cell == OR_LINEAR) {
    double a = u_in[0], b = u_in[1], h = s[0];
    s_next[0] = a * h + b;
    if (J) J[0] = a;
    if (dfdu) { dfdu[0] = h; dfdu[1] = 1.0; }
    if (wcoef) { wcoef[0] = 0.0; wcoef[1] = 0.0; }
    return OR_OK;
  }
  if (cell == OR_GRU) {
    double h = s[0];
    double z = sigmoid(u_in[0] + w[0] * h + bias[0]);
    double r = sigmoid(u_in[1] + w[1] * h + bias[1]);
    double c = tanh(u_in[2] + w[2] * (r * h) + bias[2]);
    s_next[0] = (1.0 - z) * h + z * c;
    /* partial derivatives of h' with respect to each gate pre-activation */
    double d_uz = (c - h) * z * (1.0 - z);           /* via z            */
    double d_uc = z * (1.0 - c * c);                 /* via c            */
    double d_ur = d_uc * w[2] * h * r * (1.0 - r);   /* via r inside c   */
    if (dfdu) { dfdu[0] = d_uz; dfdu[1] = d_ur; dfdu[2] = d_uc; }
    if (wcoef) { wcoef[0] = h; wcoef[1] = h; wcoef[2] = r * h; }
    if (J) {
      /* dh'/dh = (1-z) + (c-h) dz/dh + z dc/dh,
         dz/dh = z(1-z) a_z,  dc/dh = (1-c^2) a_c (r + h dr/dh),
         dr/dh = r(1-r) a_r                                            */
      double dz_dh = z * (1.0 - z) * w[0];
      double dr_dh = r * (1.0 - r) * w[1];
      double dc_dh = (1.0 - c * c) * w[2] * (r + h * dr_dh);
      J[0] = (1.0 - z) + (c - h) * dz_dh + z * dc_dh;
    }
    return OR_OK;
  }
  if (cell == OR_LSTM) {
    double c = s[0], h = s[1];
    double ig = sigmoid(u_in[0] + w[0] * h + bias[0]);
    double fg = sigmoid(u_in[1] + w[1] * h + bias[1]);
    double og = sigmoid(u_in[2] + w[2] * h + bias[2]);
    double gg = tanh(u_in[3] + w[3] * h + bias[3]);
    double c2 = fg * c + ig * gg;
    double tc = tanh(c2);
    double h2 = og * tc;
    s_next[0] = c2;
    s_next[1] = h2;
    /* d c' / d u_gate (gate order i, f, o, g); o does not enter c' */
    double dc_du[4] = {gg * ig * (1.0 - ig), c * fg * (1.0 - fg), 0.0,
                       ig * (1.0 - gg * gg)};
    double kh = og * (1.0 - tc * tc); /* d h' / d c' */
    double dh_du[4] = {kh * dc_du[0], kh * dc_du[1], tc * og * (1.0 - og),
                       kh * dc_du[3]};
    if (dfdu) {
      for (int g = 0; g < 4; ++g) { dfdu[0 * 4 + g] = dc_du[g]; dfdu[1 * 4 + g] = dh_du[g]; }
    }
    if (wcoef) { for (int g = 0; g < 4; ++g) wcoef[g] = h; }
    if (J) {
      /* every gate sees h through w_g * h, so d c'/d h = sum_g dc_du[g] w_g */
      double dc_dh = dc_du[0] * w[0] + dc_du[1] * w[1] + dc_du[3] * w[3];
      double dh_dh = dh_du[2] * w[2] + kh * dc_dh;
      J[0] = fg;        /* d c'/d c */
      J[1] = dc_dh;     /* d c'/d h */
      J[2] = kh * fg;   /* d h'/d c */
      J[3] = dh_dh;     /* d h'/d h */
    }
    return OR_OK;
  }
  if (cell == OR_SLSTM) {
    double c = s[0], n = s[1], m = s[2], h = s[3];
    double uz = u_in[0] + w[0] * h + bias[0], ui = u_in[1] + w[1] * h + bias[1];
    double uf = u_in[2] + w[2] * h + bias[2], uo = u_in[3] + w[3] * h + bias[3];
    double z = tanh(uz), o = sigmoid(uo);
    double lf = log_sigmoid(uf), dlf = sigmoid(-uf); /* d lf / d u_f */
    int fb = lf + m >= ui;                           /* the forget term sets m' */
    double m2 = fb ? lf + m : ui;
    double ip = exp(ui - m2), fp = exp(lf + m - m2);
    double c2 = fp * c + ip * z, n2 = fp * n + ip, h2 = o * c2 / n2;
    s_next[0] = c2; s_next[1] = n2; s_next[2] = m2; s_next[3] = h2;
    /* m', i', f' as functions of (u_i, u_f, m) */
    double dm_ui = fb ? 0.0 : 1.0, dm_uf = fb ? dlf : 0.0, dm_m = fb ? 1.0 : 0.0;
    double dip_ui = ip * (1.0 - dm_ui), dip_uf = -ip * dm_uf, dip_m = -ip * dm_m;
    double dfp_ui = -fp * dm_ui, dfp_uf = fp * (dlf - dm_uf), dfp_m = fp * (1.0 - dm_m);
    /* d (c', n', m') / d u_g, gate order z, i, f, o */
    double dc_du[4] = {ip * (1.0 - z * z), c * dfp_ui + z * dip_ui, c * dfp_uf + z * dip_uf, 0.0};
    double dn_du[4] = {0.0, n * dfp_ui + dip_ui, n * dfp_uf + dip_uf, 0.0};
    double dm_du[4] = {0.0, dm_ui, dm_uf, 0.0};
    double dh_du[4];
    for (int g = 0; g < 4; ++g) dh_du[g] = o * (dc_du[g] * n2 - c2 * dn_du[g]) / (n2 * n2);
    dh_du[3] += (c2 / n2) * o * (1.0 - o);
    if (dfdu) {
      for (int g = 0; g < 4; ++g) {
        dfdu[0 * 4 + g] = dc_du[g]; dfdu[1 * 4 + g] = dn_du[g];
        dfdu[2 * 4 + g] = dm_du[g]; dfdu[3 * 4 + g] = dh_du[g];
      }
    }
    if (wcoef) { for (int g = 0; g < 4; ++g) wcoef[g] = h; }
    if (J) {
      double dc_m = c * dfp_m + z * dip_m, dn_m = n * dfp_m + dip_m;
      double sc = 0.0, sn_ = 0.0, sm = 0.0, sh = 0.0; /* h enters every gate through w_g h */
      for (int g = 0; g < 4; ++g) {
        sc += dc_du[g] * w[g]; sn_ += dn_du[g] * w[g]; sm += dm_du[g] * w[g]; sh += dh_du[g] * w[g];
      }
      J[0] = fp;  J[1] = 0.0; J[2] = dc_m;  J[3] = sc;
      J[4] = 0.0; J[5] = fp;  J[6] = dn_m;  J[7] = sn_;
      J[8] = 0.0; J[9] = 0.0; J[10] = dm_m; J[11] = sm;
      J[12] = o * fp / n2;                          /* d h' / d c */
      J[13] = -o * c2 * fp / (n2 * n2);             /* d h' / d n */
      J[14] = o * (dc_m * n2 - c2 * dn_m) / (n2 * n2);
      J[15] = sh;
    }
    return OR_OK;
  }
  return OR_EINVAL;
}

/* ------------------------------------------------------------------------ */
/* problem description shared by the entry points below                     */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t cell;
  int32_t dtype;       /* storage of pre[] */
  int64_t B, T, D;
  const void* pre[4];  /* G planes [B][T][D] */
  const float* w;      /* [G][D] (GRU, LSTM)  */
  const float* bias;   /* [G][D] (GRU, LSTM)  */
  const float* s0;     /* [S][B][D] or NULL (zeros) */
  const unsigned char* seg_start; /* [T] or NULL: nonzero where a new packed sequence begins
                                     (that step's previous state is zero; s0 is the first
                                     sequence's initial state)                              */
  int64_t head_size;   /* OR_HGRU: channels per head (D = n_heads * head_size); w is then
                          [3][n_heads][head_size][head_size]; ignored by the other cells    */
} or_problem;

static int64_t elem_index(const or_problem* p, int64_t b, int64_t t, int64_t d) {
  return (b * p->T + t) * p->D + d;
}

/* gate inputs of channel (b,d) at time t, decoded to fp64 */
static void gather_u(const or_problem* p, int64_t b, int64_t t, int64_t d, double* u) {
  int G = gate_count(p->cell);
  int64_t i = elem_index(p, b, t, d);
  for (int g = 0; g < G; ++g) u[g] = load_in(p->pre[g], p->dtype, i);
}

static void gather_params(const or_problem* p, int64_t d, double* w, double* bias) {
  int G = gate_count(p->cell);
  for (int g = 0; g < G; ++g) {
    w[g] = (p->cell == OR_LINEAR) ? 0.0 : (double)p->w[g * p->D + d];
    bias[g] = (p->cell == OR_LINEAR) ? 0.0 : (double)p->bias[g * p->D + d];
  }
}

static void gather_s0(const or_problem* p, int64_t b, int64_t d, double* s) {
  int S = state_size(p->cell);
  for (int k = 0; k < S; ++k)
    s[k] = p->s0 ? (double)p->s0[(k * p->B + b) * p->D + d] : 0.0;
}

/* does step t begin a new packed sequence (t > 0)? */
static int starts_at(const or_problem* p, int64_t t) { return t > 0 && p->seg_start && p->seg_start[t]; }

/* the state step t starts from: s0 at t = 0, zero where a new sequence begins, else H_{t-1} */
static void prev_state(const or_problem* p, const double* H, int64_t b, int64_t t, int64_t d, double* prev);

/* state plane k of a trajectory laid out [S][B][T][D] */
static int64_t traj_index(const or_problem* p, int k, int64_t b, int64_t t, int64_t d) {
  return ((k * p->B + b) * p->T + t) * p->D + d;
}

static void prev_state(const or_problem* p, const double* H, int64_t b, int64_t t, int64_t d, double* prev) {
  int S = state_size(p->cell);
  if (t == 0) gather_s0(p, b, d, prev);
  else if (starts_at(p, t)) for (int k = 0; k < S; ++k) prev[k] = 0.0;
  else for (int k = 0; k < S; ++k) prev[k] = H[traj_index(p, k, b, t - 1, d)];
}

/* head-wise block GRU entry points (defined at the end of this file) */
static int hgru_unroll(const or_problem* p, double* out, int nthreads);
static int hgru_residual(const or_problem* p, const double* H, double* out_max, int nthreads);
static int hgru_newton(const or_problem* p, double* H, int picard_iters, int max_iters, double tol,
                       double* resid, int* iters, int* converged, int nthreads);
static int hgru_warm(const or_problem* p, double* H, int nthreads);
static int hgru_vjp(const or_problem* p, const double* s, const float* g, double* d_pre, double* d_w,
                    double* d_bias, double* d_s0, double* lam, int nthreads);

/* ------------------------------------------------------------------------ */
/* a tiny thread pool over channels                                          */
/* ------------------------------------------------------------------------ */

typedef void (*channel_fn)(void* ctx, int64_t ch0, int64_t ch1, int worker);

typedef struct {
  channel_fn fn;
  void* ctx;
  int64_t ch0, ch1;
  int worker;
} worker_arg;

static void* worker_main(void* a) {
  worker_arg* w = (worker_arg*)a;
  w->fn(w->ctx, w->ch0, w->ch1, w->worker);
  return NULL;
}

static int run_channels(int64_t n_channels, int nthreads, channel_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n_channels) nthreads = (int)(n_channels > 0 ? n_channels : 1);
  if (nthreads == 1) { fn(ctx, 0, n_channels, 0); return OR_OK; }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  worker_arg* args = (worker_arg*)malloc(sizeof(worker_arg) * nthreads);
  if (!th || !args) { free(th); free(args); return OR_ENOMEM; }
  for (int i = 0; i < nthreads; ++i) {
    args[i].fn = fn;
    args[i].ctx = ctx;
    args[i].ch0 = n_channels * i / nthreads;
    args[i].ch1 = n_channels * (i + 1) / nthreads;
    args[i].worker = i;
    pthread_create(&th[i], NULL, worker_main, &args[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(args);
  return OR_OK;
}

static int check_problem(const or_problem* p) {
  if (!p || p->B < 0 || p->T < 0 || p->D < 0) return OR_EINVAL;
  if (p->cell != OR_LINEAR && p->cell != OR_GRU && p->cell != OR_LSTM && p->cell != OR_SLSTM &&
      p->cell != OR_HGRU) return OR_EINVAL;
  if (p->cell == OR_HGRU && (p->head_size < 1 || p->D % p->head_size != 0)) return OR_EINVAL;
  if (p->dtype != OR_F32 && p->dtype != OR_BF16) return OR_EINVAL;
  int G = gate_count(p->cell);
  for (int g = 0; g < G; ++g)
    if (!p->pre[g] && p->B * p->T * p->D > 0) return OR_EINVAL;
  if (p->cell != OR_LINEAR && (!p->w || !p->bias) && p->D > 0) return OR_EINVAL;
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* sequential unroll: s_t = f(s_{t-1}, x_t), the exact solution of F(H)=0    */
/* ------------------------------------------------------------------------ */

typedef struct {
  const or_problem* p;
  double* out;
} unroll_ctx;

static void unroll_channels(void* vctx, int64_t ch0, int64_t ch1, int worker) {
  (void)worker;
  unroll_ctx* c = (unroll_ctx*)vctx;
  const or_problem* p = c->p;
  int S = state_size(p->cell);
  double u[OR_GMAX], w[OR_GMAX], bias[OR_GMAX], s[OR_SMAX], sn[OR_SMAX];
  for (int64_t ch = ch0; ch < ch1; ++ch) {
    int64_t b = ch / p->D, d = ch % p->D;
    gather_params(p, d, w, bias);
    gather_s0(p, b, d, s);
    for (int64_t t = 0; t < p->T; ++t) {
      if (starts_at(p, t)) for (int k = 0; k < S; ++k) s[k] = 0.0;
      gather_u(p, b, t, d, u);
      or_cell_step(p->cell, u, w, bias, s, sn, NULL, NULL, NULL);
      for (int k = 0; k < S; ++k) {
        s[k] = sn[k];
        c->out[traj_index(p, k, b, t, d)] = s[k];
      }
    }
  }
}

int or_unroll(const or_problem* p, double* out, int nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (p->cell == OR_HGRU) return hgru_unroll(p, out, nthreads);
  unroll_ctx c = {p, out};
  return run_channels(p->B * p->D, nthreads, unroll_channels, &c);
}

/* ------------------------------------------------------------------------ */
/* residual of a trajectory: max over b,t,d,state of |h_t - f(h_{t-1},x_t)|  */
/* ------------------------------------------------------------------------ */

typedef struct {
  const or_problem* p;
  const double* H;
  double* worker_max;
} resid_ctx;

/* NaN-propagating maximum: a NaN anywhere makes the result NaN */
static double nan_max(double m, double x) { return (x > m || x != x) ? x : m; }

static void resid_channels(void* vctx, int64_t ch0, int64_t ch1, int worker) {
  resid_ctx* c = (resid_ctx*)vctx;
  const or_problem* p = c->p;
  int S = state_size(p->cell);
  double u[OR_GMAX], w[OR_GMAX], bias[OR_GMAX], prev[OR_SMAX], sn[OR_SMAX], m = 0.0;
  for (int64_t ch = ch0; ch < ch1; ++ch) {
    int64_t b = ch / p->D, d = ch % p->D;
    gather_params(p, d, w, bias);
    for (int64_t t = 0; t < p->T; ++t) {
      prev_state(p, c->H, b, t, d, prev);
      gather_u(p, b, t, d, u);
      or_cell_step(p->cell, u, w, bias, prev, sn, NULL, NULL, NULL);
      for (int k = 0; k < S; ++k) m = nan_max(m, fabs(c->H[traj_index(p, k, b, t, d)] - sn[k]));
    }
  }
  c->worker_max[worker] = m;
}

int or_residual(const or_problem* p, const double* H, double* out_max, int nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (p->cell == OR_HGRU) return hgru_residual(p, H, out_max, nthreads);
  if (nthreads < 1) nthreads = 1;
  double* wm = (double*)calloc((size_t)nthreads, sizeof(double));
  if (!wm) return OR_ENOMEM;
  resid_ctx c = {p, H, wm};
  rc = run_channels(p->B * p->D, nthreads, resid_channels, &c);
  double m = 0.0;
  for (int i = 0; i < nthreads; ++i) m = nan_max(m, wm[i]);
  free(wm);
  *out_max = m;
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Newton on F(H) = 0 (pararnn-torch README, "Method")                       */
/* ------------------------------------------------------------------------ */
/*
 * Iteration k, at the current trajectory H^k (H^k_{-1} := s0; with packed
 * sequences the step before each later sequence's first is the zero state):
 *   r_t = h^k_t - f(h^k_{t-1}, x_t)                       (residual)
 *   J_t = d f / d s  at (h^k_{t-1}, x_t)                  (Jacobian)
 *   R_k = max |r_t|                                      (max residual)
 *   delta_{-1} = 0,  delta_t = J_t delta_{t-1} - r_t       (linearised system,
 *                                                          solved sequentially)
 *   H^{k+1} = H^k + delta
 * Stop rule (a reading; the pages give none): with tol <= 0 exactly max_iters
 * iterations run.  With tol > 0 the iteration whose evaluated residual R_k is
 * below tol is the last one; its update is still applied (the fused GPU pass
 * evaluates the residual and produces the update in one sweep).  A
 * non-finite R_k stops the loop and reports divergence.
 * A grown residual is divergence too (a reading: the README, "Evaluation",
 * has a divergence error carry the residual history and states no rule): with
 * tol > 0, a solve that spends its whole budget without meeting tol and whose
 * last residual R_{K-1} exceeds R_{k0}, the residual of the iterate Newton
 * started from (k0 = the number of Picard sweeps before it), ends worse than
 * it began.  Growth from one iteration to the next is not judged on its own:
 * on this triangular system Newton is exact after T updates, and on the
 * benchmark distributions the max residual of a solve that converges can
 * rise for a few iterations first (the LSTM's first update at long T, the
 * sLSTM's first Newton updates after its Picard sweeps).
 * Output: H^{iters}; resid[0..iters-1] = R_0..R_{iters-1}.
 */

typedef struct {
  const or_problem* p;
  double* H;          /* in/out trajectory [S][B][T][D] */
  double* worker_max;
  double* scratch;    /* per worker: T * (S + S*S + S) doubles */
  int picard;         /* this update is a Picard sweep: J taken as 0, so H^{k+1}_t = f(H^k_{t-1}) */
} newton_ctx;

static void newton_channels(void* vctx, int64_t ch0, int64_t ch1, int worker) {
  newton_ctx* c = (newton_ctx*)vctx;
  const or_problem* p = c->p;
  int S = state_size(p->cell);
  int64_t T = p->T;
  double* r = c->scratch + (size_t)worker * (size_t)T * (size_t)(2 * S + S * S);
  double* J = r + T * S;
  double* delta = J + T * S * S;
  double u[OR_GMAX], w[OR_GMAX], bias[OR_GMAX], prev[OR_SMAX], sn[OR_SMAX], m = 0.0;
  for (int64_t ch = ch0; ch < ch1; ++ch) {
    int64_t b = ch / p->D, d = ch % p->D;
    gather_params(p, d, w, bias);
    /* residual and Jacobian at the current iterate */
    for (int64_t t = 0; t < T; ++t) {
      prev_state(p, c->H, b, t, d, prev);
      gather_u(p, b, t, d, u);
      or_cell_step(p->cell, u, w, bias, prev, sn, J + t * S * S, NULL, NULL);
      /* where a sequence begins, h_{t-1} does not enter f: that step's Jacobian is zero; a
         Picard sweep drops the Jacobian everywhere */
      if (c->picard || starts_at(p, t)) for (int k = 0; k < S * S; ++k) J[t * S * S + k] = 0.0;
      for (int k = 0; k < S; ++k) {
        r[t * S + k] = c->H[traj_index(p, k, b, t, d)] - sn[k];
        m = nan_max(m, fabs(r[t * S + k]));
      }
    }
    /* sequential solve of the linearised recurrence */
    for (int64_t t = 0; t < T; ++t) {
      for (int i = 0; i < S; ++i) {
        double acc = -r[t * S + i];
        if (t > 0)
          for (int j = 0; j < S; ++j) acc += J[t * S * S + i * S + j] * delta[(t - 1) * S + j];
        delta[t * S + i] = acc;
      }
    }
    for (int64_t t = 0; t < T; ++t)
      for (int k = 0; k < S; ++k) c->H[traj_index(p, k, b, t, d)] += delta[t * S + k];
  }
  c->worker_max[worker] = m;
}

/* warm start (pararnn-torch README, "Method": the GRU/LSTM first iterate is the cell applied to a
   zero previous state): H^0_t = f(0, x_t) for every t */
typedef struct {
  const or_problem* p;
  double* H;
} warm_ctx;

static void warm_channels(void* vctx, int64_t ch0, int64_t ch1, int worker) {
  (void)worker;
  warm_ctx* c = (warm_ctx*)vctx;
  const or_problem* p = c->p;
  int S = state_size(p->cell);
  double u[OR_GMAX], w[OR_GMAX], bias[OR_GMAX], zero[OR_SMAX] = {0.0, 0.0, 0.0, 0.0}, sn[OR_SMAX];
  for (int64_t ch = ch0; ch < ch1; ++ch) {
    int64_t b = ch / p->D, d = ch % p->D;
    gather_params(p, d, w, bias);
    for (int64_t t = 0; t < p->T; ++t) {
      gather_u(p, b, t, d, u);
      or_cell_step(p->cell, u, w, bias, zero, sn, NULL, NULL, NULL);
      for (int k = 0; k < S; ++k) c->H[traj_index(p, k, b, t, d)] = sn[k];
    }
  }
}

/* init_mode: 0 = init_guess or zeros, 1 = warm start (ignored when init_guess is given).
   picard_iters: the first min(picard_iters, max_iters) updates are Picard (fixed-point) sweeps
   H^{k+1}_t = f(H^k_{t-1}, x_t) instead of Newton updates (pararnn-torch README, "API overview":
   Picard iterations warm the first guess for the sLSTM); they count as iterations. */
int or_newton(const or_problem* p, const float* init_guess, int init_mode, int picard_iters, int max_iters,
              double tol, double* H, double* resid, int* iters, int* converged, int nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (max_iters < 1) return OR_EINVAL;
  int S = state_size(p->cell);
  int64_t n = (int64_t)S * p->B * p->T * p->D;
  for (int64_t i = 0; i < n; ++i) H[i] = init_guess ? (double)init_guess[i] : 0.0;
  if (nthreads < 1) nthreads = 1;
  if (p->cell == OR_HGRU) {
    if (!init_guess && init_mode == 1) {
      rc = hgru_warm(p, H, nthreads);
      if (rc) return rc;
    }
    return hgru_newton(p, H, picard_iters, max_iters, tol, resid, iters, converged, nthreads);
  }
  if (!init_guess && init_mode == 1) {
    warm_ctx wc = {p, H};
    rc = run_channels(p->B * p->D, nthreads, warm_channels, &wc);
    if (rc) return rc;
  }
  double* wm = (double*)malloc(sizeof(double) * (size_t)nthreads);
  double* scratch = (double*)malloc(sizeof(double) * (size_t)nthreads *
                                    (size_t)(p->T > 0 ? p->T : 1) * (size_t)(2 * S + S * S));
  if (!wm || !scratch) { free(wm); free(scratch); return OR_ENOMEM; }
  newton_ctx c = {p, H, wm, scratch, 0};
  int k_done = 0, conv = 0, status = OR_OK;
  for (int k = 0; k < max_iters; ++k) {
    c.picard = k < picard_iters;
    for (int i = 0; i < nthreads; ++i) wm[i] = 0.0;
    rc = run_channels(p->B * p->D, nthreads, newton_channels, &c);
    if (rc) { status = rc; break; }
    double R = 0.0;
    for (int i = 0; i < nthreads; ++i) R = nan_max(R, wm[i]);
    resid[k] = R;
    k_done = k + 1;
    if (!isfinite(R)) { status = OR_DIVERGED; break; } /* NaN or Inf */
    if (tol > 0.0 && R < tol) { conv = 1; break; }
  }
  /* the budget spent without convergence, ending above the residual Newton started from */
  if (status == OR_OK && tol > 0.0 && !conv && k_done - 1 > picard_iters && resid[k_done - 1] > resid[picard_iters])
    status = OR_DIVERGED;
  free(wm);
  free(scratch);
  *iters = k_done;
  *converged = conv;
  return status;
}

/* ------------------------------------------------------------------------ */
/* linear recurrence, S = 1 or 2, forward or reverse                         */
/* ------------------------------------------------------------------------ */
/*
 * forward:  s_{-1} = s0,  s_t = A_t s_{t-1} + b_t,  t = 0..T-1
 * reverse:  s_T    = s0,  s_t = A_t s_{t+1} + b_t,  t = T-1..0
 * With packed sequences (seg_start[t] set where one begins), s_{t-1} (forward)
 * or s_{t+1} (reverse) is zero across each boundary between sequences.
 * S = 1: a is [B][T][D], b is [B][T][D].
 * S = 2: a is [4][B][T][D] (A00, A01, A10, A11 row-major), b is [2][B][T][D].
 * This is the recurrence that every Newton linear solve reduces to
 * (pararnn-torch README, "Method": the linearised system is solved by a scan along time);
 * here it is evaluated by its definition, one step after another.
 */

typedef struct {
  int S, dtype, reverse;
  int64_t B, T, D;
  const void* a;
  const void* b;
  const float* s0;
  const unsigned char* seg_start;
  double* out;
} lin_ctx;

static void lin_channels(void* vctx, int64_t ch0, int64_t ch1, int worker) {
  (void)worker;
  lin_ctx* c = (lin_ctx*)vctx;
  int64_t N = c->B * c->T * c->D;
  for (int64_t ch = ch0; ch < ch1; ++ch) {
    int64_t b = ch / c->D, d = ch % c->D;
    double s[2] = {0.0, 0.0};
    for (int k = 0; k < c->S; ++k) s[k] = c->s0 ? (double)c->s0[(k * c->B + b) * c->D + d] : 0.0;
    for (int64_t step = 0; step < c->T; ++step) {
      int64_t t = c->reverse ? c->T - 1 - step : step;
      int64_t i = (b * c->T + t) * c->D + d;
      /* packed sequences: the state entering a sequence's first step (forward) or last step
         (reverse) is zero */
      int64_t edge = c->reverse ? t + 1 : t;
      if (c->seg_start && edge > 0 && edge < c->T && c->seg_start[edge]) s[0] = s[1] = 0.0;
      if (c->S == 1) {
        s[0] = load_in(c->a, c->dtype, i) * s[0] + load_in(c->b, c->dtype, i);
        c->out[i] = s[0];
      } else {
        double a00 = load_in(c->a, c->dtype, 0 * N + i), a01 = load_in(c->a, c->dtype, 1 * N + i);
        double a10 = load_in(c->a, c->dtype, 2 * N + i), a11 = load_in(c->a, c->dtype, 3 * N + i);
        double n0 = a00 * s[0] + a01 * s[1] + load_in(c->b, c->dtype, 0 * N + i);
        double n1 = a10 * s[0] + a11 * s[1] + load_in(c->b, c->dtype, 1 * N + i);
        s[0] = n0;
        s[1] = n1;
        c->out[0 * N + i] = n0;
        c->out[1 * N + i] = n1;
      }
    }
  }
}

int or_linear_scan(int S, int64_t B, int64_t T, int64_t D, int dtype, const void* a,
                   const void* b, const float* s0, const unsigned char* seg_start, int reverse,
                   double* out, int nthreads) {
  if ((S != 1 && S != 2) || B < 0 || T < 0 || D < 0) return OR_EINVAL;
  if (dtype != OR_F32 && dtype != OR_BF16) return OR_EINVAL;
  lin_ctx c = {S, dtype, reverse ? 1 : 0, B, T, D, a, b, s0, seg_start, out};
  return run_channels(B * D, nthreads, lin_channels, &c);
}

/* ------------------------------------------------------------------------ */
/* VJP at a solved trajectory (README "Method": backward by the adjoint)     */
/* ------------------------------------------------------------------------ */
/*
 * For L with dL/dh_t = g_t given on the h component of the state:
 *   lambda_{T-1} = e_h g_{T-1}
 *   lambda_t     = e_h g_t + J_{t+1}^T lambda_{t+1}        (reverse, sequential)
 *   J_{t+1} = d f/d s at (s_t, x_{t+1})
 *   dL/du_{gate,t} = sum_i lambda_t[i] * d s_t[i] / d u_gate   at (s_{t-1}, x_t)
 *   dL/dU_{gate,t} = dL/du_{gate,t}          (U enters u additively)
 *   dL/dw_gate     = sum_{b,t} dL/du_{gate,t} * (factor of w_gate in u_gate)
 *   dL/dbias_gate  = sum_{b,t} dL/du_{gate,t}
 *   dL/ds0         = J_0^T lambda_0,  J_0 = d f/d s at (s0, x_0)
 * LINEAR: dL/da_t = lambda_t h_{t-1}, dL/db_t = lambda_t, dL/ds0 = a_0 lambda_0.
 * Packed sequences: J_{t+1} is taken as zero where step t+1 begins a sequence
 * (no adjoint flows back across it), and s_{t-1} is zero at such a step.
 * e_h is the unit vector of h (for the LSTM state (c, h), e_h = (0, 1)).
 * Sums over (b, t) are accumulated in plain sequential order per channel.
 */

typedef struct {
  const or_problem* p;
  const double* s;    /* trajectory [S][B][T][D] */
  const float* g;     /* [B][T][D] */
  double* d_pre;      /* [G][B][T][D] */
  double* lam;        /* [S][B][T][D] or NULL */
  double* d_s0;       /* [S][B][D] or NULL */
  double* wpart;      /* [B*D][G] per-channel sums of dL/dw */
  double* bpart;      /* [B*D][G] per-channel sums of dL/dbias */
  double* scratch;    /* per worker: T * S doubles */
} vjp_ctx;

static void vjp_channels(void* vctx, int64_t ch0, int64_t ch1, int worker) {
  vjp_ctx* c = (vjp_ctx*)vctx;
  const or_problem* p = c->p;
  int S = state_size(p->cell), G = gate_count(p->cell);
  int64_t T = p->T, N = p->B * p->T * p->D;
  double* lam = c->scratch + (size_t)worker * (size_t)T * (size_t)S;
  double u[OR_GMAX], w[OR_GMAX], bias[OR_GMAX], prev[OR_SMAX], sn[OR_SMAX], J[OR_SMAX * OR_SMAX];
  double dfdu[OR_SMAX * OR_GMAX], wcoef[OR_GMAX];
  for (int64_t ch = ch0; ch < ch1; ++ch) {
    int64_t b = ch / p->D, d = ch % p->D;
    gather_params(p, d, w, bias);
    /* adjoint recurrence, backwards in time */
    for (int64_t t = T - 1; t >= 0; --t) {
      double acc[OR_SMAX] = {0.0, 0.0, 0.0, 0.0};
      acc[S - 1] = (double)c->g[elem_index(p, b, t, d)]; /* e_h g_t */
      if (t + 1 < T && !starts_at(p, t + 1)) {   /* nothing flows back across a sequence start */
        for (int k = 0; k < S; ++k) prev[k] = c->s[traj_index(p, k, b, t, d)];
        gather_u(p, b, t + 1, d, u);
        or_cell_step(p->cell, u, w, bias, prev, sn, J, NULL, NULL);
        for (int i = 0; i < S; ++i)            /* (J^T lambda)_i = sum_j J[j][i] lambda_j */
          for (int j = 0; j < S; ++j) acc[i] += J[j * S + i] * lam[(t + 1) * S + j];
      }
      for (int i = 0; i < S; ++i) lam[t * S + i] = acc[i];
    }
    /* gate gradients and parameter sums, forwards in time */
    double wsum[4] = {0, 0, 0, 0}, bsum[4] = {0, 0, 0, 0};
    for (int64_t t = 0; t < T; ++t) {
      prev_state(p, c->s, b, t, d, prev);
      gather_u(p, b, t, d, u);
      or_cell_step(p->cell, u, w, bias, prev, sn, J, dfdu, wcoef);
      for (int gi = 0; gi < G; ++gi) {
        double du = 0.0;
        for (int i = 0; i < S; ++i) du += lam[t * S + i] * dfdu[i * G + gi];
        c->d_pre[gi * N + elem_index(p, b, t, d)] = du;
        wsum[gi] += du * wcoef[gi];
        bsum[gi] += du;
      }
      if (c->lam)
        for (int k = 0; k < S; ++k) c->lam[traj_index(p, k, b, t, d)] = lam[t * S + k];
      if (t == 0 && c->d_s0) {
        for (int i = 0; i < S; ++i) {
          double acc = 0.0;
          for (int j = 0; j < S; ++j) acc += J[j * S + i] * lam[0 * S + j];
          c->d_s0[(i * p->B + b) * p->D + d] = acc;
        }
      }
    }
    if (T == 0 && c->d_s0)
      for (int i = 0; i < S; ++i) c->d_s0[(i * p->B + b) * p->D + d] = 0.0;
    for (int gi = 0; gi < G; ++gi) {
      c->wpart[ch * G + gi] = wsum[gi];
      c->bpart[ch * G + gi] = bsum[gi];
    }
  }
}

int or_vjp(const or_problem* p, const double* s, const float* g, double* d_pre, double* d_w,
           double* d_bias, double* d_s0, double* lam, int nthreads) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (p->cell == OR_HGRU) return hgru_vjp(p, s, g, d_pre, d_w, d_bias, d_s0, lam, nthreads);
  int S = state_size(p->cell), G = gate_count(p->cell);
  int64_t C = p->B * p->D;
  if (nthreads < 1) nthreads = 1;
  double* wpart = (double*)calloc((size_t)(C > 0 ? C : 1) * (size_t)G, sizeof(double));
  double* bpart = (double*)calloc((size_t)(C > 0 ? C : 1) * (size_t)G, sizeof(double));
  double* scratch = (double*)malloc(sizeof(double) * (size_t)nthreads *
                                    (size_t)(p->T > 0 ? p->T : 1) * (size_t)S);
  if (!wpart || !bpart || !scratch) { free(wpart); free(bpart); free(scratch); return OR_ENOMEM; }
  vjp_ctx c = {p, s, g, d_pre, lam, d_s0, wpart, bpart, scratch};
  rc = run_channels(C, nthreads, vjp_channels, &c);
  /* parameter gradients: sum over batch of the per-channel sums (b ascending) */
  if (rc == OR_OK && p->cell != OR_LINEAR) {
    for (int gi = 0; gi < G; ++gi) {
      for (int64_t d = 0; d < p->D; ++d) {
        double ws = 0.0, bs = 0.0;
        for (int64_t b = 0; b < p->B; ++b) {
          ws += wpart[(b * p->D + d) * G + gi];
          bs += bpart[(b * p->D + d) * G + gi];
        }
        if (d_w) d_w[gi * p->D + d] = ws;
        if (d_bias) d_bias[gi * p->D + d] = bs;
      }
    }
  }
  free(wpart);
  free(bpart);
  free(scratch);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* head-wise block GRU                                                        */
/* ------------------------------------------------------------------------ */
/*
 * pararnn-torch README, "Usage" (Dreamer-style block GRU: ParaGRU with
 * the head-wise mixing mode and a head count; block-diagonal recurrent matrices, factorized Newton) and "News"
 * (factorized Newton for that cell).  The page prints no equations.  Reading:
 * the channels split into n_heads heads of hs = D / n_heads consecutive
 * channels; each gate's recurrent matrix A_g is block-diagonal with one dense
 * hs x hs block per head, and otherwise the cell is the diagonal GRU above
 * with A_g in place of the diagonal weight (A_c acts on r * h):
 *   z = sig(U_z + A_z h + b_z),  r = sig(U_r + A_r h + b_r),
 *   c = tanh(U_c + A_c (r * h) + b_c),  h' = (1 - z) * h + z * c
 * (hs = 1 is the diagonal GRU).  Heads do not interact, so F(H) = 0 and its
 * Newton system split into one block-bidiagonal system per (batch row, head)
 * with dense hs x hs Jacobian blocks: that split is read as the
 * "factorization".  Newton uses the exact block Jacobian.
 * Layout: w = [3][n_heads][hs][hs], block row i = output channel, column j =
 * input channel; bias = [3][D]; gate order z, r, c.
 */

static int64_t hgru_heads(const or_problem* p) { return p->D / p->head_size; }

/* One step of one head in fp64.  u = 3*hs gate inputs, A = [3][hs][hs], bias = 3*hs, h = hs.
   Outputs: hn[hs]; optional J[hs*hs] (J[i*hs+j] = d hn_i / d h_j), dz[hs] = d hn_i / d u_z,i,
   dc[hs] = d hn_i / d u_c,i, dr[hs*hs] (dr[i*hs+k] = d hn_i / d u_r,k), rh[hs] = r_j h_j (the
   vector A_c multiplies).  Caller-provided work space: none (hs <= OR_HMAX). */
enum { OR_HMAX = 256 };
int or_hgru_step(int64_t hs, const double* u, const double* A, const double* bias, const double* h,
                 double* hn, double* J, double* dz, double* dc, double* dr, double* rh) {
  if (hs < 1 || hs > OR_HMAX) return OR_EINVAL;
  const double *Az = A, *Ar = A + hs * hs, *Ac = A + 2 * hs * hs;
  double z[OR_HMAX], r[OR_HMAX], c[OR_HMAX], rv[OR_HMAX], pz[OR_HMAX], pc[OR_HMAX];
  for (int64_t i = 0; i < hs; ++i) {
    double az = 0.0, ar = 0.0;
    for (int64_t j = 0; j < hs; ++j) {
      az += Az[i * hs + j] * h[j];
      ar += Ar[i * hs + j] * h[j];
    }
    z[i] = sigmoid(u[i] + az + bias[i]);
    r[i] = sigmoid(u[hs + i] + ar + bias[hs + i]);
  }
  for (int64_t j = 0; j < hs; ++j) rv[j] = r[j] * h[j];
  for (int64_t i = 0; i < hs; ++i) {
    double ac = 0.0;
    for (int64_t j = 0; j < hs; ++j) ac += Ac[i * hs + j] * rv[j];
    c[i] = tanh(u[2 * hs + i] + ac + bias[2 * hs + i]);
    hn[i] = (1.0 - z[i]) * h[i] + z[i] * c[i];
    pz[i] = (c[i] - h[i]) * z[i] * (1.0 - z[i]);   /* via z_i            */
    pc[i] = z[i] * (1.0 - c[i] * c[i]);            /* via c_i            */
  }
  if (dz) for (int64_t i = 0; i < hs; ++i) dz[i] = pz[i];
  if (dc) for (int64_t i = 0; i < hs; ++i) dc[i] = pc[i];
  if (rh) for (int64_t j = 0; j < hs; ++j) rh[j] = rv[j];
  /* u_r,k moves h'_i through c_i: d u_c,i / d u_r,k = A_c[i][k] h_k r_k (1 - r_k) */
  if (dr)
    for (int64_t i = 0; i < hs; ++i)
      for (int64_t k = 0; k < hs; ++k) dr[i * hs + k] = pc[i] * Ac[i * hs + k] * h[k] * r[k] * (1.0 - r[k]);
  if (J) {
    /* d h'_i / d h_j = (1 - z_i) [i = j] + (c_i - h_i) z_i (1 - z_i) A_z[i][j]
                        + z_i (1 - c_i^2) d u_c,i / d h_j,
       d u_c,i / d h_j = A_c[i][j] r_j + sum_k A_c[i][k] h_k r_k (1 - r_k) A_r[k][j] */
    for (int64_t i = 0; i < hs; ++i) {
      for (int64_t j = 0; j < hs; ++j) {
        double duc = Ac[i * hs + j] * r[j];
        for (int64_t k = 0; k < hs; ++k) duc += Ac[i * hs + k] * h[k] * r[k] * (1.0 - r[k]) * Ar[k * hs + j];
        J[i * hs + j] = (i == j ? 1.0 - z[i] : 0.0) + pz[i] * Az[i * hs + j] + pc[i] * duc;
      }
    }
  }
  return OR_OK;
}

/* a chain is one (batch row, head): ch = b * n_heads + head */
static void hgru_params(const or_problem* p, int64_t head, double* A, double* bias) {
  const int64_t hs = p->head_size, H = hgru_heads(p);
  for (int g = 0; g < 3; ++g) {
    for (int64_t i = 0; i < hs * hs; ++i) A[g * hs * hs + i] = (double)p->w[(g * H + head) * hs * hs + i];
    for (int64_t i = 0; i < hs; ++i) bias[g * hs + i] = (double)p->bias[g * p->D + head * hs + i];
  }
}

static void hgru_gather(const or_problem* p, int64_t b, int64_t t, int64_t head, double* u) {
  const int64_t hs = p->head_size;
  for (int g = 0; g < 3; ++g)
    for (int64_t i = 0; i < hs; ++i) u[g * hs + i] = load_in(p->pre[g], p->dtype, elem_index(p, b, t, head * hs + i));
}

/* the state step t of chain (b, head) starts from: s0, zero at a sequence start, else H_{t-1} */
static void hgru_prev(const or_problem* p, const double* H, int64_t b, int64_t t, int64_t head, double* prev) {
  const int64_t hs = p->head_size;
  for (int64_t i = 0; i < hs; ++i) {
    const int64_t d = head * hs + i;
    if (t == 0) prev[i] = p->s0 ? (double)p->s0[b * p->D + d] : 0.0;
    else if (starts_at(p, t)) prev[i] = 0.0;
    else prev[i] = H[elem_index(p, b, t - 1, d)];
  }
}

/* per-worker buffers of one chain walk */
typedef struct {
  double *A, *bias, *u, *prev, *hn, *J, *dz, *dc, *dr, *rh, *old, *delta, *lam, *tmp;
} hgru_buf;

static int hgru_buf_alloc(hgru_buf* w, int64_t hs, int64_t T, int want_lam) {
  const size_t v = (size_t)hs, m = (size_t)(hs * hs);
  double* base = (double*)malloc(sizeof(double) * (3 * m + 3 * v + 3 * v + 10 * v + 2 * m +
                                                   (want_lam ? (size_t)(T > 0 ? T : 1) * v : 0)));
  if (!base) return OR_ENOMEM;
  double* q = base;
  w->A = q; q += 3 * m;
  w->bias = q; q += 3 * v;
  w->u = q; q += 3 * v;
  w->prev = q; q += v;
  w->hn = q; q += v;
  w->dz = q; q += v;
  w->dc = q; q += v;
  w->rh = q; q += v;
  w->old = q; q += v;
  w->delta = q; q += v;
  w->tmp = q; q += 3 * v;
  w->J = q; q += m;
  w->dr = q; q += m;
  w->lam = want_lam ? q : NULL;
  return OR_OK;
}

typedef struct {
  const or_problem* p;
  double* H;           /* trajectory [B][T][D] (in/out where it applies) */
  const double* Hc;    /* read-only trajectory */
  double* worker_max;
  int picard;
  int status;
} hgru_ctx;

static void hgru_unroll_chains(void* vctx, int64_t c0, int64_t c1, int worker) {
  (void)worker;
  hgru_ctx* c = (hgru_ctx*)vctx;
  const or_problem* p = c->p;
  const int64_t hs = p->head_size, H = hgru_heads(p);
  hgru_buf w;
  if (hgru_buf_alloc(&w, hs, p->T, 0)) { c->status = OR_ENOMEM; return; }
  for (int64_t ch = c0; ch < c1; ++ch) {
    const int64_t b = ch / H, head = ch % H;
    hgru_params(p, head, w.A, w.bias);
    for (int64_t t = 0; t < p->T; ++t) {
      hgru_prev(p, c->H, b, t, head, w.prev);
      hgru_gather(p, b, t, head, w.u);
      or_hgru_step(hs, w.u, w.A, w.bias, w.prev, w.hn, NULL, NULL, NULL, NULL, NULL);
      for (int64_t i = 0; i < hs; ++i) c->H[elem_index(p, b, t, head * hs + i)] = w.hn[i];
    }
  }
  free(w.A);
}

static int hgru_unroll(const or_problem* p, double* out, int nthreads) {
  hgru_ctx c = {p, out, NULL, NULL, 0, OR_OK};
  int rc = run_channels(p->B * hgru_heads(p), nthreads, hgru_unroll_chains, &c);
  return rc ? rc : c.status;
}

static void hgru_resid_chains(void* vctx, int64_t c0, int64_t c1, int worker) {
  hgru_ctx* c = (hgru_ctx*)vctx;
  const or_problem* p = c->p;
  const int64_t hs = p->head_size, H = hgru_heads(p);
  hgru_buf w;
  if (hgru_buf_alloc(&w, hs, p->T, 0)) { c->status = OR_ENOMEM; return; }
  double m = 0.0;
  for (int64_t ch = c0; ch < c1; ++ch) {
    const int64_t b = ch / H, head = ch % H;
    hgru_params(p, head, w.A, w.bias);
    for (int64_t t = 0; t < p->T; ++t) {
      hgru_prev(p, c->Hc, b, t, head, w.prev);
      hgru_gather(p, b, t, head, w.u);
      or_hgru_step(hs, w.u, w.A, w.bias, w.prev, w.hn, NULL, NULL, NULL, NULL, NULL);
      for (int64_t i = 0; i < hs; ++i) m = nan_max(m, fabs(c->Hc[elem_index(p, b, t, head * hs + i)] - w.hn[i]));
    }
  }
  c->worker_max[worker] = m;
  free(w.A);
}

static int hgru_residual(const or_problem* p, const double* Hv, double* out_max, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  double* wm = (double*)calloc((size_t)nthreads, sizeof(double));
  if (!wm) return OR_ENOMEM;
  hgru_ctx c = {p, NULL, Hv, wm, 0, OR_OK};
  int rc = run_channels(p->B * hgru_heads(p), nthreads, hgru_resid_chains, &c);
  double m = 0.0;
  for (int i = 0; i < nthreads; ++i) m = nan_max(m, wm[i]);
  free(wm);
  *out_max = m;
  return rc ? rc : c.status;
}

/* Newton iteration k on each chain, as in or_newton: r_t = h^k_t - f(h^k_{t-1}, x_t), J_t the
   dense hs x hs block, delta_{-1} = 0, delta_t = J_t delta_{t-1} - r_t (solved sequentially),
   H^{k+1} = H^k + delta.  The walk goes forward in t and keeps the old h^k_{t-1} aside, so the
   residual and Jacobian of every step are taken at the old iterate. */
static void hgru_newton_chains(void* vctx, int64_t c0, int64_t c1, int worker) {
  hgru_ctx* c = (hgru_ctx*)vctx;
  const or_problem* p = c->p;
  const int64_t hs = p->head_size, H = hgru_heads(p);
  hgru_buf w;
  if (hgru_buf_alloc(&w, hs, p->T, 0)) { c->status = OR_ENOMEM; return; }
  double m = 0.0;
  for (int64_t ch = c0; ch < c1; ++ch) {
    const int64_t b = ch / H, head = ch % H;
    hgru_params(p, head, w.A, w.bias);
    for (int64_t t = 0; t < p->T; ++t) {
      /* the previous state at the OLD iterate: s0, zero at a sequence start, else old h_{t-1} */
      if (t == 0 || starts_at(p, t)) hgru_prev(p, c->H, b, t, head, w.prev);
      else for (int64_t i = 0; i < hs; ++i) w.prev[i] = w.old[i];
      hgru_gather(p, b, t, head, w.u);
      or_hgru_step(hs, w.u, w.A, w.bias, w.prev, w.hn, w.J, NULL, NULL, NULL, NULL);
      const int no_jac = c->picard || starts_at(p, t);   /* as in or_newton: J = 0 there */
      for (int64_t i = 0; i < hs; ++i) {
        const int64_t e = elem_index(p, b, t, head * hs + i);
        const double r = c->H[e] - w.hn[i];
        m = nan_max(m, fabs(r));
        double acc = -r;
        if (t > 0 && !no_jac)
          for (int64_t j = 0; j < hs; ++j) acc += w.J[i * hs + j] * w.delta[j];
        w.tmp[i] = acc;
      }
      for (int64_t i = 0; i < hs; ++i) {
        const int64_t e = elem_index(p, b, t, head * hs + i);
        w.old[i] = c->H[e];
        w.delta[i] = w.tmp[i];
        c->H[e] += w.delta[i];
      }
    }
  }
  c->worker_max[worker] = m;
  free(w.A);
}

static int hgru_newton(const or_problem* p, double* Hv, int picard_iters, int max_iters, double tol,
                       double* resid, int* iters, int* converged, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  double* wm = (double*)malloc(sizeof(double) * (size_t)nthreads);
  if (!wm) return OR_ENOMEM;
  hgru_ctx c = {p, Hv, NULL, wm, 0, OR_OK};
  int k_done = 0, conv = 0, status = OR_OK;
  for (int k = 0; k < max_iters; ++k) {
    c.picard = k < picard_iters;
    for (int i = 0; i < nthreads; ++i) wm[i] = 0.0;
    int rc = run_channels(p->B * hgru_heads(p), nthreads, hgru_newton_chains, &c);
    if (rc || c.status) { status = rc ? rc : c.status; break; }
    double R = 0.0;
    for (int i = 0; i < nthreads; ++i) R = nan_max(R, wm[i]);
    resid[k] = R;
    k_done = k + 1;
    if (!isfinite(R)) { status = OR_DIVERGED; break; }
    if (tol > 0.0 && R < tol) { conv = 1; break; }
  }
  /* the budget spent without convergence, ending above the residual Newton started from (or_newton) */
  if (status == OR_OK && tol > 0.0 && !conv && k_done - 1 > picard_iters && resid[k_done - 1] > resid[picard_iters])
    status = OR_DIVERGED;
  free(wm);
  *iters = k_done;
  *converged = conv;
  return status;
}

/* warm start: H^0_t = f(0, x_t) */
static void hgru_warm_chains(void* vctx, int64_t c0, int64_t c1, int worker) {
  (void)worker;
  hgru_ctx* c = (hgru_ctx*)vctx;
  const or_problem* p = c->p;
  const int64_t hs = p->head_size, H = hgru_heads(p);
  hgru_buf w;
  if (hgru_buf_alloc(&w, hs, p->T, 0)) { c->status = OR_ENOMEM; return; }
  for (int64_t i = 0; i < hs; ++i) w.prev[i] = 0.0;
  for (int64_t ch = c0; ch < c1; ++ch) {
    const int64_t b = ch / H, head = ch % H;
    hgru_params(p, head, w.A, w.bias);
    for (int64_t t = 0; t < p->T; ++t) {
      hgru_gather(p, b, t, head, w.u);
      or_hgru_step(hs, w.u, w.A, w.bias, w.prev, w.hn, NULL, NULL, NULL, NULL, NULL);
      for (int64_t i = 0; i < hs; ++i) c->H[elem_index(p, b, t, head * hs + i)] = w.hn[i];
    }
  }
  free(w.A);
}

static int hgru_warm(const or_problem* p, double* Hv, int nthreads) {
  hgru_ctx c = {p, Hv, NULL, NULL, 0, OR_OK};
  int rc = run_channels(p->B * hgru_heads(p), nthreads, hgru_warm_chains, &c);
  return rc ? rc : c.status;
}

/* VJP, as or_vjp with dense blocks: lambda_{T-1} = g_{T-1}, lambda_t = g_t + J_{t+1}^T lambda_{t+1}
   (zero across a sequence start); then per step
     dU_z,i = lambda_i dz_i,  dU_c,i = lambda_i dc_i,  dU_r,k = sum_i lambda_i dr[i][k],
     dA_z[i][j] += dU_z,i h_j,  dA_r[i][j] += dU_r,i h_j,  dA_c[i][j] += dU_c,i (r h)_j,
     dbias_g,i += dU_g,i     (h = the step's previous state),
   dL/ds0 = J_0^T lambda_0.  Sums: per chain in t order, then over b ascending per head. */
typedef struct {
  const or_problem* p;
  const double* s;
  const float* g;
  double* d_pre;     /* [3][B][T][D] */
  double* lam;       /* [B][T][D] or NULL */
  double* d_s0;      /* [B][D] or NULL */
  double* apart;     /* [B*H][3][hs][hs] */
  double* bpart;     /* [B*H][3][hs] */
  int status;
} hgru_vjp_ctx;

static void hgru_vjp_chains(void* vctx, int64_t c0, int64_t c1, int worker) {
  (void)worker;
  hgru_vjp_ctx* c = (hgru_vjp_ctx*)vctx;
  const or_problem* p = c->p;
  const int64_t hs = p->head_size, H = hgru_heads(p), T = p->T, N = p->B * p->T * p->D;
  hgru_buf w;
  if (hgru_buf_alloc(&w, hs, T, 1)) { c->status = OR_ENOMEM; return; }
  for (int64_t ch = c0; ch < c1; ++ch) {
    const int64_t b = ch / H, head = ch % H;
    hgru_params(p, head, w.A, w.bias);
    for (int64_t t = T - 1; t >= 0; --t) {
      for (int64_t i = 0; i < hs; ++i) w.tmp[i] = (double)c->g[elem_index(p, b, t, head * hs + i)];
      if (t + 1 < T && !starts_at(p, t + 1)) {
        for (int64_t i = 0; i < hs; ++i) w.prev[i] = c->s[elem_index(p, b, t, head * hs + i)];
        hgru_gather(p, b, t + 1, head, w.u);
        or_hgru_step(hs, w.u, w.A, w.bias, w.prev, w.hn, w.J, NULL, NULL, NULL, NULL);
        for (int64_t i = 0; i < hs; ++i)        /* (J^T lambda)_i = sum_j J[j][i] lambda_j */
          for (int64_t j = 0; j < hs; ++j) w.tmp[i] += w.J[j * hs + i] * w.lam[(t + 1) * hs + j];
      }
      for (int64_t i = 0; i < hs; ++i) w.lam[t * hs + i] = w.tmp[i];
    }
    double* ap = c->apart + ch * 3 * hs * hs;
    double* bp = c->bpart + ch * 3 * hs;
    for (int64_t i = 0; i < 3 * hs * hs; ++i) ap[i] = 0.0;
    for (int64_t i = 0; i < 3 * hs; ++i) bp[i] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      hgru_prev(p, c->s, b, t, head, w.prev);
      hgru_gather(p, b, t, head, w.u);
      or_hgru_step(hs, w.u, w.A, w.bias, w.prev, w.hn, w.J, w.dz, w.dc, w.dr, w.rh);
      const double* lam = w.lam + t * hs;
      double* du = w.tmp;   /* du[g*hs + i] */
      for (int64_t i = 0; i < hs; ++i) {
        du[i] = lam[i] * w.dz[i];
        du[2 * hs + i] = lam[i] * w.dc[i];
        double acc = 0.0;
        for (int64_t k = 0; k < hs; ++k) acc += lam[k] * w.dr[k * hs + i];
        du[hs + i] = acc;
      }
      for (int g = 0; g < 3; ++g) {
        const double* x = (g == 2) ? w.rh : w.prev;   /* the vector A_g multiplies */
        for (int64_t i = 0; i < hs; ++i) {
          const int64_t e = elem_index(p, b, t, head * hs + i);
          c->d_pre[g * N + e] = du[g * hs + i];
          bp[g * hs + i] += du[g * hs + i];
          for (int64_t j = 0; j < hs; ++j) ap[(g * hs + i) * hs + j] += du[g * hs + i] * x[j];
        }
      }
      if (c->lam)
        for (int64_t i = 0; i < hs; ++i) c->lam[elem_index(p, b, t, head * hs + i)] = lam[i];
      if (t == 0 && c->d_s0)
        for (int64_t i = 0; i < hs; ++i) {
          double acc = 0.0;
          for (int64_t j = 0; j < hs; ++j) acc += w.J[j * hs + i] * lam[j];
          c->d_s0[b * p->D + head * hs + i] = acc;
        }
    }
    if (T == 0 && c->d_s0)
      for (int64_t i = 0; i < hs; ++i) c->d_s0[b * p->D + head * hs + i] = 0.0;
  }
  free(w.A);
}

static int hgru_vjp(const or_problem* p, const double* s, const float* g, double* d_pre, double* d_w,
                    double* d_bias, double* d_s0, double* lam, int nthreads) {
  const int64_t hs = p->head_size, H = hgru_heads(p), C = p->B * H;
  double* apart = (double*)calloc((size_t)(C > 0 ? C : 1) * 3 * (size_t)(hs * hs), sizeof(double));
  double* bpart = (double*)calloc((size_t)(C > 0 ? C : 1) * 3 * (size_t)hs, sizeof(double));
  if (!apart || !bpart) { free(apart); free(bpart); return OR_ENOMEM; }
  hgru_vjp_ctx c = {p, s, g, d_pre, lam, d_s0, apart, bpart, OR_OK};
  int rc = run_channels(C, nthreads, hgru_vjp_chains, &c);
  if (!rc) rc = c.status;
  if (rc == OR_OK) {
    for (int gi = 0; gi < 3; ++gi)
      for (int64_t head = 0; head < H; ++head) {
        for (int64_t e = 0; e < hs * hs; ++e) {
          double acc = 0.0;
          for (int64_t b = 0; b < p->B; ++b) acc += apart[((b * H + head) * 3 + gi) * hs * hs + e];
          if (d_w) d_w[(gi * H + head) * hs * hs + e] = acc;
        }
        for (int64_t i = 0; i < hs; ++i) {
          double acc = 0.0;
          for (int64_t b = 0; b < p->B; ++b) acc += bpart[((b * H + head) * 3 + gi) * hs + i];
          if (d_bias) d_bias[gi * p->D + head * hs + i] = acc;
        }
      }
  }
  free(apart);
  free(bpart);
  return rc;
}

/* ABI version of this file's entry points, so the wrapper can check it */
int or_abi_version(void) { return 7; }
