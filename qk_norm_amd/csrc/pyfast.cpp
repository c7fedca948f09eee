/* Python entry points of the QK-Norm C ABI with no argument-conversion layer.
 *
 * Two kinds of call, both argument marshalling only (every step of the work
 * runs in libqknorm.so):
 * - per_head, layerwise, partial_sumsq, apply_scalar and the qkv_proj_per_head
 *   calls (plain, _ws, _noalloc) take the C ABI's arguments as Python ints and floats
 *   (pointers as ints, 0 or None for NULL), convert them to C values and call the library's
 *   extern "C" function, returning its int status.  They replace ctypes,
 *   whose per-call conversion of eleven or more arguments costs about a
 *   microsecond, a third of a decode-sized launch.
 * - per_head_t and layerwise_t take the binding's own arguments (torch
 *   tensors) and read from them what the binding's Python path would, through
 *   torch's C++ tensor API (no Python-level attribute calls, each of which
 *   costs about 0.1 us): the common case only, and None for anything else
 *   (see below).
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stdint.h>

#include <torch/csrc/autograd/python_variable.h>

#include "../../include/qknorm.h"

static int as_ptr(PyObject* o, void** out) {
  if (o == Py_None) {
    *out = NULL;
    return 0;
  }
  const unsigned long long v = PyLong_AsUnsignedLongLong(o);
  if (v == (unsigned long long)-1 && PyErr_Occurred()) return -1;
  *out = (void*)(uintptr_t)v;
  return 0;
}

static int as_i64(PyObject* o, int64_t* out) {
  const long long v = PyLong_AsLongLong(o);
  if (v == -1 && PyErr_Occurred()) return -1;
  *out = (int64_t)v;
  return 0;
}

static int as_i32(PyObject* o, int32_t* out) {
  const long v = PyLong_AsLong(o);
  if (v == -1 && PyErr_Occurred()) return -1;
  if (v < INT32_MIN || v > INT32_MAX) {
    PyErr_SetString(PyExc_OverflowError, "argument does not fit a 32-bit int");
    return -1;
  }
  *out = (int32_t)v;
  return 0;
}

static int as_f32(PyObject* o, float* out) {
  const double v = PyFloat_AsDouble(o);
  if (v == -1.0 && PyErr_Occurred()) return -1;
  *out = (float)v;
  return 0;
}

static int nargs_ok(Py_ssize_t n, Py_ssize_t want, const char* name) {
  if (n == want) return 1;
  PyErr_Format(PyExc_TypeError, "%s takes %zd arguments (%zd given)", name, want, n);
  return 0;
}

/* per_head(qkv, T, ld, hq, hkv, head_dim, gamma_q, gamma_k, eps, dtype, stream) -> int */
static PyObject* f_per_head(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  void *qkv, *gq, *gk, *st;
  int64_t T, ld;
  int32_t hq, hkv, d, dt;
  float eps;
  if (!nargs_ok(n, 11, "per_head")) return NULL;
  if (as_ptr(a[0], &qkv) || as_i64(a[1], &T) || as_i64(a[2], &ld) || as_i32(a[3], &hq) ||
      as_i32(a[4], &hkv) || as_i32(a[5], &d) || as_ptr(a[6], &gq) || as_ptr(a[7], &gk) ||
      as_f32(a[8], &eps) || as_i32(a[9], &dt) || as_ptr(a[10], &st))
    return NULL;
  return PyLong_FromLong(qknorm_per_head(qkv, T, ld, hq, hkv, d, gq, gk, eps, dt, st));
}

/* layerwise(qkv, T, ld, wq, wk, gamma_q, gamma_k, eps, nshards, dtype, stream) -> int */
static PyObject* f_layerwise(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  void *qkv, *gq, *gk, *st;
  int64_t T, ld, wq, wk;
  int32_t ns, dt;
  float eps;
  if (!nargs_ok(n, 11, "layerwise")) return NULL;
  if (as_ptr(a[0], &qkv) || as_i64(a[1], &T) || as_i64(a[2], &ld) || as_i64(a[3], &wq) ||
      as_i64(a[4], &wk) || as_ptr(a[5], &gq) || as_ptr(a[6], &gk) || as_f32(a[7], &eps) ||
      as_i32(a[8], &ns) || as_i32(a[9], &dt) || as_ptr(a[10], &st))
    return NULL;
  return PyLong_FromLong(qknorm_layerwise(qkv, T, ld, wq, wk, gq, gk, eps, ns, dt, st));
}

/* partial_sumsq(qkv, T, ld, wq, wk, nshards, part_q, part_k, dtype, stream) -> int */
static PyObject* f_partial_sumsq(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  void *qkv, *pq, *pk, *st;
  int64_t T, ld, wq, wk;
  int32_t ns, dt;
  if (!nargs_ok(n, 10, "partial_sumsq")) return NULL;
  if (as_ptr(a[0], &qkv) || as_i64(a[1], &T) || as_i64(a[2], &ld) || as_i64(a[3], &wq) ||
      as_i64(a[4], &wk) || as_i32(a[5], &ns) || as_ptr(a[6], &pq) || as_ptr(a[7], &pk) ||
      as_i32(a[8], &dt) || as_ptr(a[9], &st))
    return NULL;
  return PyLong_FromLong(qknorm_partial_sumsq(qkv, T, ld, wq, wk, ns, (float*)pq, (float*)pk, dt, st));
}

/* apply_scalar(qkv, T, ld, wq, wk, part_q, part_k, nparts, norm_wq, norm_wk, gamma_q, gamma_k,
 *              eps, dtype, stream) -> int */
static PyObject* f_apply_scalar(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  void *qkv, *pq, *pk, *gq, *gk, *st;
  int64_t T, ld, wq, wk, nwq, nwk;
  int32_t np, dt;
  float eps;
  if (!nargs_ok(n, 15, "apply_scalar")) return NULL;
  if (as_ptr(a[0], &qkv) || as_i64(a[1], &T) || as_i64(a[2], &ld) || as_i64(a[3], &wq) ||
      as_i64(a[4], &wk) || as_ptr(a[5], &pq) || as_ptr(a[6], &pk) || as_i32(a[7], &np) ||
      as_i64(a[8], &nwq) || as_i64(a[9], &nwk) || as_ptr(a[10], &gq) || as_ptr(a[11], &gk) ||
      as_f32(a[12], &eps) || as_i32(a[13], &dt) || as_ptr(a[14], &st))
    return NULL;
  return PyLong_FromLong(qknorm_apply_scalar(qkv, T, ld, wq, wk, (const float*)pq, (const float*)pk,
                                             np, nwq, nwk, gq, gk, eps, dt, st));
}

/* qkv_proj_per_head(x, ldx, w, ldw, qkv, ld, T, hidden, hq, hkv, head_dim, gamma_q, gamma_k, eps,
 *                   flags, dtype, stream) -> int */
static PyObject* f_qkv_proj_per_head(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  void *x, *w, *qkv, *gq, *gk, *st;
  int64_t ldx, ldw, ld, T, hidden;
  int32_t hq, hkv, d, fl, dt;
  float eps;
  if (!nargs_ok(n, 17, "qkv_proj_per_head")) return NULL;
  if (as_ptr(a[0], &x) || as_i64(a[1], &ldx) || as_ptr(a[2], &w) || as_i64(a[3], &ldw) ||
      as_ptr(a[4], &qkv) || as_i64(a[5], &ld) || as_i64(a[6], &T) || as_i64(a[7], &hidden) ||
      as_i32(a[8], &hq) || as_i32(a[9], &hkv) || as_i32(a[10], &d) || as_ptr(a[11], &gq) ||
      as_ptr(a[12], &gk) || as_f32(a[13], &eps) || as_i32(a[14], &fl) || as_i32(a[15], &dt) ||
      as_ptr(a[16], &st))
    return NULL;
  return PyLong_FromLong(
      qknorm_qkv_proj_per_head(x, ldx, w, ldw, qkv, ld, T, hidden, hq, hkv, d, gq, gk, eps, fl, dt, st));
}

/* qkv_proj_per_head_noalloc: the arguments of qkv_proj_per_head -> int */
static PyObject* f_qkv_proj_per_head_noalloc(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  void *x, *w, *qkv, *gq, *gk, *st;
  int64_t ldx, ldw, ld, T, hidden;
  int32_t hq, hkv, d, fl, dt;
  float eps;
  if (!nargs_ok(n, 17, "qkv_proj_per_head_noalloc")) return NULL;
  if (as_ptr(a[0], &x) || as_i64(a[1], &ldx) || as_ptr(a[2], &w) || as_i64(a[3], &ldw) ||
      as_ptr(a[4], &qkv) || as_i64(a[5], &ld) || as_i64(a[6], &T) || as_i64(a[7], &hidden) ||
      as_i32(a[8], &hq) || as_i32(a[9], &hkv) || as_i32(a[10], &d) || as_ptr(a[11], &gq) ||
      as_ptr(a[12], &gk) || as_f32(a[13], &eps) || as_i32(a[14], &fl) || as_i32(a[15], &dt) ||
      as_ptr(a[16], &st))
    return NULL;
  return PyLong_FromLong(qknorm_qkv_proj_per_head_noalloc(x, ldx, w, ldw, qkv, ld, T, hidden, hq, hkv,
                                                          d, gq, gk, eps, fl, dt, st));
}

/* qkv_proj_per_head_ws(x, ldx, w, ldw, qkv, ld, T, hidden, hq, hkv, head_dim, gamma_q, gamma_k,
 *                      eps, flags, dtype, workspace, workspace_bytes, stream) -> int */
static PyObject* f_qkv_proj_per_head_ws(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  void *x, *w, *qkv, *gq, *gk, *ws, *st;
  int64_t ldx, ldw, ld, T, hidden, wsb;
  int32_t hq, hkv, d, fl, dt;
  float eps;
  if (!nargs_ok(n, 19, "qkv_proj_per_head_ws")) return NULL;
  if (as_ptr(a[0], &x) || as_i64(a[1], &ldx) || as_ptr(a[2], &w) || as_i64(a[3], &ldw) ||
      as_ptr(a[4], &qkv) || as_i64(a[5], &ld) || as_i64(a[6], &T) || as_i64(a[7], &hidden) ||
      as_i32(a[8], &hq) || as_i32(a[9], &hkv) || as_i32(a[10], &d) || as_ptr(a[11], &gq) ||
      as_ptr(a[12], &gk) || as_f32(a[13], &eps) || as_i32(a[14], &fl) || as_i32(a[15], &dt) ||
      as_ptr(a[16], &ws) || as_i64(a[17], &wsb) || as_ptr(a[18], &st))
    return NULL;
  return PyLong_FromLong(qknorm_qkv_proj_per_head_ws(x, ldx, w, ldw, qkv, ld, T, hidden, hq, hkv, d, gq,
                                                     gk, eps, fl, dt, ws, wsb, st));
}

/* ------------------------------------------------------------------------
 * The common case of the binding's marshalling, on torch tensors: qkv a
 * contiguous [T, ...] GPU torch.Tensor (T > 0; not a subclass) of a dtype the
 * library takes, gamma None or a contiguous torch.Tensor on the same GPU in
 * the dtype that goes with qkv's.  The same facts the Python binding reads
 * (device, dtype, contiguity, rows, data pointer), read from the tensor's
 * C++ object.  Anything else returns None, and the binding's Python path
 * handles it (views with a row pitch, and every error, with its message).
 * `setup` hands over torch's current-raw-stream function and the
 * torch.Tensor type. */

static PyObject* g_tensor;          /* torch.Tensor: only that exact type takes the C++ path */
static PyObject* g_raw_stream;      /* torch._C._cuda_getCurrentRawStream; set last, so that
                                       its presence means the rest is ready */

static PyObject* f_setup(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  if (!nargs_ok(n, 2, "setup")) return NULL;
  if (!PyType_Check(a[1])) {
    PyErr_SetString(PyExc_TypeError, "setup(raw_stream, tensor_type)");
    return NULL;
  }
  Py_XSETREF(g_tensor, Py_NewRef(a[1]));
  Py_XSETREF(g_raw_stream, Py_NewRef(a[0]));
  Py_RETURN_NONE;
}

/* The tensor inside o when o is exactly a torch.Tensor, else NULL. */
static const at::Tensor* tensor_of(PyObject* o) {
  if ((PyObject*)Py_TYPE(o) != g_tensor) return NULL;
  return &THPVariable_Unpack(o);
}

/* The library's dtype code of a tensor, or -1 for another dtype. */
static int dtype_code(const at::Tensor& t) {
  switch (t.scalar_type()) {
    case c10::ScalarType::Float: return QKNORM_F32;
    case c10::ScalarType::BFloat16: return QKNORM_BF16;
    case c10::ScalarType::Half: return QKNORM_F16;
    case c10::ScalarType::Float8_e4m3fn: return QKNORM_FP8_E4M3;
    default: return -1;
  }
}

/* qkv: 1 and (T, ld, dev, ptr, code) for the common case, 0 otherwise */
static int qkv_rows(PyObject* o, int64_t* T, int64_t* ld, int64_t* dev, void** ptr, int* code) {
  const at::Tensor* t = tensor_of(o);
  if (!t || !t->is_cuda() || (*code = dtype_code(*t)) < 0 || !t->is_contiguous() || t->dim() < 2) return 0;
  *T = t->size(0);
  if (*T <= 0) return 0;
  *ld = t->numel() / *T;
  *dev = t->get_device();
  *ptr = t->data_ptr();
  return 1;
}

/* gamma: 1 and its pointer (NULL for None) for the common case, 0 otherwise;
 * the dtype that goes with qkv's is its own, bf16 for FP8 */
static int gamma_ptr(PyObject* g, int code, int64_t dev, void** ptr) {
  if (g == Py_None) {
    *ptr = NULL;
    return 1;
  }
  const at::Tensor* t = tensor_of(g);
  const int want = code == QKNORM_FP8_E4M3 ? QKNORM_BF16 : code;
  if (!t || dtype_code(*t) != want || !t->is_contiguous() || !t->is_cuda() || t->get_device() != dev)
    return 0;
  *ptr = t->data_ptr();
  return 1;
}

/* the stream handle: torch's current raw stream on `dev` for None, else
 * `stream.cuda_stream` or the int itself */
static int stream_ptr(PyObject* s, int64_t dev, void** out) {
  PyObject* v;
  if (s == Py_None) {
    PyObject* d = PyLong_FromLongLong(dev);
    if (!d) return -1;
    v = PyObject_CallOneArg(g_raw_stream, d);
    Py_DECREF(d);
  } else if (PyLong_Check(s)) {
    v = Py_NewRef(s);
  } else {
    v = PyObject_GetAttrString(s, "cuda_stream");
  }
  if (!v) return -1;
  const int r = as_ptr(v, out);
  Py_DECREF(v);
  return r;
}

/* per_head_t(qkv, hq, hkv, head_dim, gamma_q, gamma_k, eps, stream) -> int or None */
static PyObject* f_per_head_t(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  if (!nargs_ok(n, 8, "per_head_t")) return NULL;
  if (!g_raw_stream) Py_RETURN_NONE;
  int64_t T, ld, dev;
  void *qkv, *gq, *gk, *st;
  int code;
  int32_t hq, hkv, d;
  float eps;
  if (!qkv_rows(a[0], &T, &ld, &dev, &qkv, &code) || !gamma_ptr(a[4], code, dev, &gq) ||
      !gamma_ptr(a[5], code, dev, &gk))
    Py_RETURN_NONE;
  if (as_i32(a[1], &hq) || as_i32(a[2], &hkv) || as_i32(a[3], &d) || as_f32(a[6], &eps) ||
      stream_ptr(a[7], dev, &st))
    return NULL;
  return PyLong_FromLong(qknorm_per_head(qkv, T, ld, hq, hkv, d, gq, gk, eps, code, st));
}

/* layerwise_t(qkv, wq, wk, gamma_q, gamma_k, eps, nshards, stream) -> int or None */
static PyObject* f_layerwise_t(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  if (!nargs_ok(n, 8, "layerwise_t")) return NULL;
  if (!g_raw_stream) Py_RETURN_NONE;
  int64_t T, ld, dev, wq, wk;
  void *qkv, *gq, *gk, *st;
  int code;
  int32_t ns;
  float eps;
  if (!qkv_rows(a[0], &T, &ld, &dev, &qkv, &code) || !gamma_ptr(a[3], code, dev, &gq) ||
      !gamma_ptr(a[4], code, dev, &gk))
    Py_RETURN_NONE;
  if (as_i64(a[1], &wq) || as_i64(a[2], &wk) || as_f32(a[5], &eps) || as_i32(a[6], &ns) ||
      stream_ptr(a[7], dev, &st))
    return NULL;
  return PyLong_FromLong(qknorm_layerwise(qkv, T, ld, wq, wk, gq, gk, eps, ns, code, st));
}

static PyMethodDef kMethods[] = {
    {"setup", (PyCFunction)(void (*)(void))f_setup, METH_FASTCALL,
     "hand over torch's current-raw-stream function and the torch.Tensor type"},
    {"per_head_t", (PyCFunction)(void (*)(void))f_per_head_t, METH_FASTCALL,
     "qknorm_per_head on torch tensors (common case; None: use the Python path)"},
    {"layerwise_t", (PyCFunction)(void (*)(void))f_layerwise_t, METH_FASTCALL,
     "qknorm_layerwise on torch tensors (common case; None: use the Python path)"},
    {"per_head", (PyCFunction)(void (*)(void))f_per_head, METH_FASTCALL, "qknorm_per_head"},
    {"layerwise", (PyCFunction)(void (*)(void))f_layerwise, METH_FASTCALL, "qknorm_layerwise"},
    {"partial_sumsq", (PyCFunction)(void (*)(void))f_partial_sumsq, METH_FASTCALL, "qknorm_partial_sumsq"},
    {"apply_scalar", (PyCFunction)(void (*)(void))f_apply_scalar, METH_FASTCALL, "qknorm_apply_scalar"},
    {"qkv_proj_per_head", (PyCFunction)(void (*)(void))f_qkv_proj_per_head, METH_FASTCALL,
     "qknorm_qkv_proj_per_head"},
    {"qkv_proj_per_head_ws", (PyCFunction)(void (*)(void))f_qkv_proj_per_head_ws, METH_FASTCALL,
     "qknorm_qkv_proj_per_head_ws"},
    {"qkv_proj_per_head_noalloc", (PyCFunction)(void (*)(void))f_qkv_proj_per_head_noalloc,
     METH_FASTCALL, "qknorm_qkv_proj_per_head_noalloc"},
    {NULL, NULL, 0, NULL}};

static struct PyModuleDef kModule = {PyModuleDef_HEAD_INIT, "_qknorm_fast",
                                     "Direct calls of the QK-Norm C ABI (see qk_norm_amd).", -1,
                                     kMethods, NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__qknorm_fast(void) { return PyModule_Create(&kModule); }
