/* tk_py.c -- the CPython extension module `_tkpy`: argument marshalling from
 * Python objects to the C ABI of include/tk.h, one function per entry point
 * under the same name.  Nothing else happens here: every function converts its
 * arguments and calls the library.
 *
 * Conversions:
 *   pointer  None -> NULL; int -> that address; any other object -> the int
 *            its data_ptr() returns (a torch tensor).
 *   stream   None -> the stream returned by the getter set with
 *            _set_stream_getter (the package sets torch's current stream);
 *            int -> that handle; other -> its cuda_stream attribute.
 *   integers and floats as Python's int() / float() would take them.
 * Every function returns the tk_status code as a Python int.
 *
 * It exists because a ctypes call with eleven arguments costs about as much
 * host time as a small launch takes on the GPU; a decode-sized launch issued
 * from Python is then bound by the binding, not by the kernel.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>

#include "tk.h"

static PyObject* g_stream_getter = NULL; /* callable returning a stream handle */

static int as_ptr(PyObject* o, void* out)
{
    void** p = (void**)out;
    if (o == Py_None) {
        *p = NULL;
        return 1;
    }
    if (PyLong_Check(o)) {
        *p = PyLong_AsVoidPtr(o);
        return !PyErr_Occurred();
    }
    PyObject* r = PyObject_CallMethod(o, "data_ptr", NULL);
    if (!r)
        return 0;
    *p = PyLong_AsVoidPtr(r);
    Py_DECREF(r);
    return !PyErr_Occurred();
}

static int as_stream(PyObject* o, void* out)
{
    void** p = (void**)out;
    if (PyLong_Check(o)) {
        *p = PyLong_AsVoidPtr(o);
        return !PyErr_Occurred();
    }
    PyObject* h = NULL;
    if (o == Py_None) {
        if (!g_stream_getter) {
            *p = NULL;
            return 1;
        }
        h = PyObject_CallNoArgs(g_stream_getter);
    } else {
        h = PyObject_GetAttrString(o, "cuda_stream");
    }
    if (!h)
        return 0;
    *p = PyLong_AsVoidPtr(h);
    Py_DECREF(h);
    return !PyErr_Occurred();
}

static PyObject* status(tk_status rc) { return PyLong_FromLong((long)rc); }

/* Run one library call without the GIL (the library never calls back into
 * Python; other threads can issue their own launches meanwhile, as they could
 * through ctypes). */
#define TK_CALL(rc, expr)              \
    do {                               \
        Py_BEGIN_ALLOW_THREADS rc = (expr); \
        Py_END_ALLOW_THREADS           \
    } while (0)

static PyObject* py_set_stream_getter(PyObject* self, PyObject* fn)
{
    (void)self;
    if (fn != Py_None && !PyCallable_Check(fn)) {
        PyErr_SetString(PyExc_TypeError, "stream getter must be callable or None");
        return NULL;
    }
    Py_XINCREF(fn == Py_None ? NULL : fn);
    Py_XDECREF(g_stream_getter);
    g_stream_getter = fn == Py_None ? NULL : fn;
    Py_RETURN_NONE;
}

static PyObject* py_tk_init(PyObject* self, PyObject* args)
{
    (void)self;
    int device;
    if (!PyArg_ParseTuple(args, "i", &device))
        return NULL;
    tk_status rc;
    TK_CALL(rc, tk_init(device));
    return status(rc);
}

static PyObject* py_tk_status_str(PyObject* self, PyObject* args)
{
    (void)self;
    int code;
    if (!PyArg_ParseTuple(args, "i", &code))
        return NULL;
    return PyUnicode_FromString(tk_status_str((tk_status)code));
}

typedef tk_status (*swiglu_cast_fn)(const void*, const float*, int64_t, int64_t, int64_t, float, tk_scale_fmt, void*,
                                    void*, int64_t*, void*);

static PyObject* swiglu_cast(swiglu_cast_fn fn, PyObject* args)
{
    void *x, *w, *codes, *scales, *count, *stream = NULL;
    long long n, hidden, group;
    float clamp;
    int sfmt;
    PyObject* so = Py_None;
    if (!PyArg_ParseTuple(args, "O&O&LLLfiO&O&O&|O", as_ptr, &x, as_ptr, &w, &n, &hidden, &group, &clamp, &sfmt,
                          as_ptr, &codes, as_ptr, &scales, as_ptr, &count, &so))
        return NULL;
    if (!as_stream(so, &stream))
        return NULL;
    tk_status rc;
    TK_CALL(rc, fn(x, (const float*)w, n, hidden, group, clamp, (tk_scale_fmt)sfmt, codes, scales, (int64_t*)count,
                   stream));
    return status(rc);
}

static PyObject* py_tk_swiglu_cast_fp8(PyObject* self, PyObject* args)
{
    (void)self;
    return swiglu_cast(tk_swiglu_cast_fp8, args);
}

static PyObject* py_tk_swiglu_cast_fp4(PyObject* self, PyObject* args)
{
    (void)self;
    return swiglu_cast(tk_swiglu_cast_fp4, args);
}

static PyObject* py_tk_swiglu_forward(PyObject* self, PyObject* args)
{
    (void)self;
    void *x, *w, *y, *count, *stream = NULL;
    long long n, hidden;
    float clamp;
    PyObject* so = Py_None;
    if (!PyArg_ParseTuple(args, "O&O&LLfO&O&|O", as_ptr, &x, as_ptr, &w, &n, &hidden, &clamp, as_ptr, &y, as_ptr,
                          &count, &so))
        return NULL;
    if (!as_stream(so, &stream))
        return NULL;
    tk_status rc;
    TK_CALL(rc, tk_swiglu_forward(x, (const float*)w, n, hidden, clamp, (float*)y, (int64_t*)count, stream));
    return status(rc);
}

typedef tk_status (*cast_fn)(const void*, tk_dtype, int64_t, int64_t, int64_t, tk_scale_fmt, void*, void*, void*);

static PyObject* cast(cast_fn fn, PyObject* args)
{
    void *x, *codes, *scales, *stream = NULL;
    int in_dtype, sfmt;
    long long n, hidden, group;
    PyObject* so = Py_None;
    if (!PyArg_ParseTuple(args, "O&iLLLiO&O&|O", as_ptr, &x, &in_dtype, &n, &hidden, &group, &sfmt, as_ptr, &codes,
                          as_ptr, &scales, &so))
        return NULL;
    if (!as_stream(so, &stream))
        return NULL;
    tk_status rc;
    TK_CALL(rc, fn(x, (tk_dtype)in_dtype, n, hidden, group, (tk_scale_fmt)sfmt, codes, scales, stream));
    return status(rc);
}

static PyObject* py_tk_cast_fp8(PyObject* self, PyObject* args)
{
    (void)self;
    return cast(tk_cast_fp8, args);
}

static PyObject* py_tk_cast_fp4(PyObject* self, PyObject* args)
{
    (void)self;
    return cast(tk_cast_fp4, args);
}

static PyObject* py_tk_topk_gate(PyObject* self, PyObject* args)
{
    (void)self;
    void *scores, *idx, *w, *stream = NULL;
    long long tokens, experts, k, n_group, topk_group;
    int normalise;
    PyObject* so = Py_None;
    if (!PyArg_ParseTuple(args, "O&LLLLLpO&O&|O", as_ptr, &scores, &tokens, &experts, &k, &n_group, &topk_group,
                          &normalise, as_ptr, &idx, as_ptr, &w, &so))
        return NULL;
    if (!as_stream(so, &stream))
        return NULL;
    tk_status rc;
    TK_CALL(rc, tk_topk_gate((const float*)scores, tokens, experts, k, n_group, topk_group, normalise, (int32_t*)idx,
                             (float*)w, stream));
    return status(rc);
}

static PyObject* py_tk_topk_to_pos(PyObject* self, PyObject* args)
{
    (void)self;
    void *idx, *pos, *off, *stream = NULL;
    long long tokens, k, experts;
    PyObject* so = Py_None;
    if (!PyArg_ParseTuple(args, "O&LLLO&O&|O", as_ptr, &idx, &tokens, &k, &experts, as_ptr, &pos, as_ptr, &off, &so))
        return NULL;
    if (!as_stream(so, &stream))
        return NULL;
    tk_status rc;
    TK_CALL(rc, tk_topk_to_pos((const int32_t*)idx, tokens, k, experts, (int32_t*)pos, (int32_t*)off, stream));
    return status(rc);
}

static PyObject* py_tk_moe_reduce(PyObject* self, PyObject* args)
{
    (void)self;
    void *x, *row_scale, *pos, *w, *out, *stream = NULL;
    float global_scale;
    long long tokens, k, hidden, n_rows;
    int out_dtype;
    PyObject* so = Py_None;
    if (!PyArg_ParseTuple(args, "O&O&O&O&fLLLLiO&|O", as_ptr, &x, as_ptr, &row_scale, as_ptr, &pos, as_ptr, &w,
                          &global_scale, &tokens, &k, &hidden, &n_rows, &out_dtype, as_ptr, &out, &so))
        return NULL;
    if (!as_stream(so, &stream))
        return NULL;
    tk_status rc;
    TK_CALL(rc, tk_moe_reduce(x, (const float*)row_scale, (const int32_t*)pos, (const float*)w, global_scale, tokens,
                              k, hidden, n_rows, (tk_dtype)out_dtype, out, stream));
    return status(rc);
}

static PyMethodDef kMethods[] = {
    {"_set_stream_getter", py_set_stream_getter, METH_O, "set the callable that supplies the default stream"},
    {"tk_init", py_tk_init, METH_VARARGS, "tk_init(device)"},
    {"tk_status_str", py_tk_status_str, METH_VARARGS, "tk_status_str(code)"},
    {"tk_swiglu_cast_fp8", py_tk_swiglu_cast_fp8, METH_VARARGS,
     "tk_swiglu_cast_fp8(x, topk_weight, n, hidden, group_size, clamp_limit, scale_fmt, codes, scales, "
     "clamped_count, stream=None)"},
    {"tk_swiglu_cast_fp4", py_tk_swiglu_cast_fp4, METH_VARARGS,
     "tk_swiglu_cast_fp4(x, topk_weight, n, hidden, group_size, clamp_limit, scale_fmt, codes, scales, "
     "clamped_count, stream=None)"},
    {"tk_swiglu_forward", py_tk_swiglu_forward, METH_VARARGS,
     "tk_swiglu_forward(x, topk_weight, n, hidden, clamp_limit, y, clamped_count, stream=None)"},
    {"tk_cast_fp8", py_tk_cast_fp8, METH_VARARGS,
     "tk_cast_fp8(x, in_dtype, n, hidden, group_size, scale_fmt, codes, scales, stream=None)"},
    {"tk_cast_fp4", py_tk_cast_fp4, METH_VARARGS,
     "tk_cast_fp4(x, in_dtype, n, hidden, group_size, scale_fmt, codes, scales, stream=None)"},
    {"tk_topk_gate", py_tk_topk_gate, METH_VARARGS,
     "tk_topk_gate(scores, tokens, experts, k, n_group, topk_group, normalise, topk_idx, topk_weight, stream=None)"},
    {"tk_moe_reduce", py_tk_moe_reduce, METH_VARARGS,
     "tk_moe_reduce(x, row_scale, pos, topk_weight, global_scale, tokens, k, hidden, n_rows, out_dtype, out, "
     "stream=None)"},
    {"tk_topk_to_pos", py_tk_topk_to_pos, METH_VARARGS,
     "tk_topk_to_pos(topk_idx, tokens, k, experts, pos, expert_offsets, stream=None)"},
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef kModule = {PyModuleDef_HEAD_INIT, "_tkpy", "Argument marshalling to the C ABI of tk.h.", -1,
                                     kMethods, NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__tkpy(void) { return PyModule_Create(&kModule); }
