/* Python entry points of the QK-Norm C ABI with no argument-conversion layer.
 *
 * Two kinds of call, both argument marshalling only (every step of the work
 * runs in libqknorm.so):
 * - per_head, layerwise, partial_sumsq, apply_scalar, qkv_proj_per_head take
 *   the C ABI's arguments as Python ints and floats (pointers as ints, 0 or
 *   None for NULL), convert them to C values and call the library's
 *   extern "C" function, returning its int status.  They replace ctypes,
 *   whose per-call conversion of eleven or more arguments costs about a
 *   microsecond, a third of a decode-sized launch.
 * - per_head_t and layerwise_t take the binding's own arguments (torch
 *   tensors) and read from them, in C, what the binding's Python path would:
 *   the common case only, and None for anything else (see below).
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stdint.h>

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

/* ------------------------------------------------------------------------
 * The common case of the binding's marshalling, on torch tensors: qkv a
 * contiguous [T, ...] GPU torch.Tensor (T > 0; not a subclass) of a dtype the
 * library takes, gamma
 * None or contiguous on the same GPU in the dtype that goes with qkv's.  The
 * same reads of the tensors the Python binding makes (is_cuda, dtype,
 * contiguity, device, data pointer), made from C.  Anything else returns
 * None, and the binding's Python path handles it (views with a row pitch,
 * and every error, with its message).  `setup` hands over the four torch
 * dtypes with their codes and gamma dtypes, torch's current-raw-stream
 * function and the torch.Tensor type. */

static PyObject* g_dtypes[4];       /* torch dtype objects, indexed by code */
static PyObject* g_gdtypes[4];      /* gamma dtype for each */
static PyObject* g_tensor;          /* torch.Tensor: only that exact type takes the C path */
static PyObject* g_raw_stream;      /* torch._C._cuda_getCurrentRawStream; set last, so that
                                       its presence means the rest is ready */
static PyObject *s_is_cuda, *s_dtype, *s_is_contiguous, *s_dim, *s_size, *s_numel, *s_get_device,
    *s_data_ptr;

static PyObject* f_setup(PyObject* self, PyObject* const* a, Py_ssize_t n) {
  (void)self;
  if (!nargs_ok(n, 4, "setup")) return NULL;
  if (!PyTuple_Check(a[0]) || PyTuple_GET_SIZE(a[0]) != 4 || !PyTuple_Check(a[1]) ||
      PyTuple_GET_SIZE(a[1]) != 4 || !PyType_Check(a[3])) {
    PyErr_SetString(PyExc_TypeError, "setup(dtypes[4], gamma_dtypes[4], raw_stream, tensor_type)");
    return NULL;
  }
#define INTERN(v, txt) \
  if (!v && !(v = PyUnicode_InternFromString(txt))) return NULL;
  INTERN(s_is_cuda, "is_cuda")
  INTERN(s_dtype, "dtype")
  INTERN(s_is_contiguous, "is_contiguous")
  INTERN(s_dim, "dim")
  INTERN(s_size, "size")
  INTERN(s_numel, "numel")
  INTERN(s_get_device, "get_device")
  INTERN(s_data_ptr, "data_ptr")
#undef INTERN
  for (int i = 0; i < 4; ++i) {
    Py_XSETREF(g_dtypes[i], Py_NewRef(PyTuple_GET_ITEM(a[0], i)));
    Py_XSETREF(g_gdtypes[i], Py_NewRef(PyTuple_GET_ITEM(a[1], i)));
  }
  Py_XSETREF(g_tensor, Py_NewRef(a[3]));
  Py_XSETREF(g_raw_stream, Py_NewRef(a[2]));
  Py_RETURN_NONE;
}

static int is_tensor(PyObject* o) { return (PyObject*)Py_TYPE(o) == g_tensor; }

/* 1 true, 0 false, -1 error (a Python exception is set) */
static int attr_true(PyObject* o, PyObject* name) {
  PyObject* v = PyObject_GetAttr(o, name);
  if (!v) return -1;
  const int r = PyObject_IsTrue(v);
  Py_DECREF(v);
  return r;
}

static int call_true(PyObject* o, PyObject* name) {
  PyObject* v = PyObject_CallMethodNoArgs(o, name);
  if (!v) return -1;
  const int r = PyObject_IsTrue(v);
  Py_DECREF(v);
  return r;
}

static int call_i64(PyObject* o, PyObject* name, PyObject* arg, int64_t* out) {
  PyObject* v = arg ? PyObject_CallMethodOneArg(o, name, arg) : PyObject_CallMethodNoArgs(o, name);
  if (!v) return -1;
  const long long r = PyLong_AsLongLong(v);
  Py_DECREF(v);
  if (r == -1 && PyErr_Occurred()) return -1;
  *out = r;
  return 0;
}

/* The dtype code of o (0..3), 4 for another dtype, -1 on error. */
static int dtype_code(PyObject* o) {
  PyObject* d = PyObject_GetAttr(o, s_dtype);
  if (!d) return -1;
  int code = 4;
  for (int i = 0; i < 4; ++i)
    if (d == g_dtypes[i]) code = i;
  Py_DECREF(d);
  return code;
}

/* qkv: 1 and (T, ld, dev, ptr, code) for the common case, 0 otherwise, -1 on error */
static int qkv_rows(PyObject* t, int64_t* T, int64_t* ld, int64_t* dev, void** ptr, int* code) {
  if (!is_tensor(t)) return 0;
  int r = attr_true(t, s_is_cuda);
  if (r <= 0) return r;
  if ((*code = dtype_code(t)) < 0) return -1;
  if (*code > 3) return 0;
  if ((r = call_true(t, s_is_contiguous)) <= 0) return r;
  int64_t dim, numel;
  if (call_i64(t, s_dim, NULL, &dim)) return -1;
  if (dim < 2) return 0;
  PyObject* zero = PyLong_FromLong(0);
  if (!zero) return -1;
  r = call_i64(t, s_size, zero, T);
  Py_DECREF(zero);
  if (r) return -1;
  if (*T <= 0) return 0;
  if (call_i64(t, s_numel, NULL, &numel) || call_i64(t, s_get_device, NULL, dev)) return -1;
  *ld = numel / *T;
  int64_t p;
  if (call_i64(t, s_data_ptr, NULL, &p)) return -1;
  *ptr = (void*)(uintptr_t)p;
  return 1;
}

/* gamma: 1 and its pointer (NULL for None) for the common case, 0 otherwise, -1 on error */
static int gamma_ptr(PyObject* g, int code, int64_t dev, void** ptr) {
  if (g == Py_None) {
    *ptr = NULL;
    return 1;
  }
  if (!is_tensor(g)) return 0;
  PyObject* d = PyObject_GetAttr(g, s_dtype);
  if (!d) return -1;
  const int same = d == g_gdtypes[code];
  Py_DECREF(d);
  if (!same) return 0;
  int r;
  if ((r = call_true(g, s_is_contiguous)) <= 0) return r;
  if ((r = attr_true(g, s_is_cuda)) <= 0) return r;
  int64_t gd, p;
  if (call_i64(g, s_get_device, NULL, &gd)) return -1;
  if (gd != dev) return 0;
  if (call_i64(g, s_data_ptr, NULL, &p)) return -1;
  *ptr = (void*)(uintptr_t)p;
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
  int code, r;
  int32_t hq, hkv, d;
  float eps;
  if ((r = qkv_rows(a[0], &T, &ld, &dev, &qkv, &code)) <= 0) {
    if (r < 0) return NULL;
    Py_RETURN_NONE;
  }
  if ((r = gamma_ptr(a[4], code, dev, &gq)) <= 0 || (r = gamma_ptr(a[5], code, dev, &gk)) <= 0) {
    if (r < 0) return NULL;
    Py_RETURN_NONE;
  }
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
  int code, r;
  int32_t ns;
  float eps;
  if ((r = qkv_rows(a[0], &T, &ld, &dev, &qkv, &code)) <= 0) {
    if (r < 0) return NULL;
    Py_RETURN_NONE;
  }
  if ((r = gamma_ptr(a[3], code, dev, &gq)) <= 0 || (r = gamma_ptr(a[4], code, dev, &gk)) <= 0) {
    if (r < 0) return NULL;
    Py_RETURN_NONE;
  }
  if (as_i64(a[1], &wq) || as_i64(a[2], &wk) || as_f32(a[5], &eps) || as_i32(a[6], &ns) ||
      stream_ptr(a[7], dev, &st))
    return NULL;
  return PyLong_FromLong(qknorm_layerwise(qkv, T, ld, wq, wk, gq, gk, eps, ns, code, st));
}

static PyMethodDef kMethods[] = {
    {"setup", (PyCFunction)(void (*)(void))f_setup, METH_FASTCALL, "hand over torch's dtypes and stream query"},
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
    {NULL, NULL, 0, NULL}};

static struct PyModuleDef kModule = {PyModuleDef_HEAD_INIT, "_qknorm_fast",
                                     "Direct calls of the QK-Norm C ABI (see qk_norm_amd).", -1,
                                     kMethods, NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__qknorm_fast(void) { return PyModule_Create(&kModule); }
