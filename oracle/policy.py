"""diffusion_step_policy: fail-closed validation and per-step precision.

Test infrastructure only (see the package docstring).

[DF-14664] "Behavior" and [TRT-17476] "Denoising-step activation precision":
the checkpoint publishes quantization_config.runtime.diffusion_step_policy;
the first and last scheduler steps it names run W8A16, the rest W8A8; the
choice is a pure function of the step index so CFG cond/uncond agree; a
one-step schedule stays native (W8A8); the understanding tower (reasoner)
is not step-gated, the policy states its mode outright; a checkpoint with
no policy (runtime: null) runs W8A8 on every step. Unknown or missing
fields, schema_version other than 1 and any other value of type,
index_space, default_mode or overlap are refused; overlap is validated and
not acted on.

Readings (the pages print the field names but not every value):
  * JSON form:
      {"schema_version": 1, "type": "first_last_steps",
       "index_space": "scheduler_step", "default_mode": "w8a8",
       "overlap": "a16", "first_steps": F, "last_steps": L,
       "reasoner": "a16" | "a8"}
  * index_space "scheduler_step" counts steps from 0 ([DF-15170] "Describe
    the bug": the 3+3 policy's first W8A8 step is "step 3 of 8").
  * The last-steps count is called last_steps; F and L are integers >= 0.
  * overlap "a16": where the two windows meet, the step runs 16-bit, which
    is what the predicate yields anyway.
  * The one-step carve-out is read as: num_steps == 1 runs W8A8.
"""

W8A8 = "W8A8"
W8A16 = "W8A16"

FIELDS = (
    "schema_version",
    "type",
    "index_space",
    "default_mode",
    "overlap",
    "first_steps",
    "last_steps",
    "reasoner",
)


class PolicyError(ValueError):
    pass


def _is_int(v):
    return isinstance(v, int) and not isinstance(v, bool)


def validate(policy):
    """Raise PolicyError unless `policy` is exactly the supported shape."""
    if not isinstance(policy, dict):
        raise PolicyError("policy must be a JSON object")
    unknown = sorted(set(policy) - set(FIELDS))
    if unknown:
        raise PolicyError("unknown policy fields: %s" % unknown)
    missing = [f for f in FIELDS if f not in policy]
    if missing:
        raise PolicyError("missing policy fields: %s" % missing)
    if not _is_int(policy["schema_version"]) or policy["schema_version"] != 1:
        raise PolicyError("schema_version must be 1")
    expected = {
        "type": "first_last_steps",
        "index_space": "scheduler_step",
        "default_mode": "w8a8",
        "overlap": "a16",
    }
    for key, value in expected.items():
        if policy[key] != value:
            raise PolicyError("unsupported %s: %r" % (key, policy[key]))
    for key in ("first_steps", "last_steps"):
        if not _is_int(policy[key]) or policy[key] < 0:
            raise PolicyError("%s must be an integer >= 0" % key)
    if policy["reasoner"] not in ("a16", "a8"):
        raise PolicyError("unsupported reasoner mode: %r" % (policy["reasoner"],))


def step_mode(policy, tower, step, num_steps):
    """Mode ('W8A8' or 'W8A16') of one transformer call.

    tower is 'generation' or 'reasoner'; step is the 0-based scheduler step
    and num_steps the schedule length. policy None means no policy.
    """
    if tower not in ("generation", "reasoner"):
        raise ValueError("tower must be 'generation' or 'reasoner'")
    if not (isinstance(num_steps, int) and num_steps >= 1 and 0 <= step < num_steps):
        raise ValueError("need 0 <= step < num_steps")
    if policy is None:
        return W8A8
    validate(policy)
    if tower == "reasoner":
        return W8A16 if policy["reasoner"] == "a16" else W8A8
    if num_steps == 1:
        return W8A8
    if step < policy["first_steps"] or step >= num_steps - policy["last_steps"]:
        return W8A16
    return W8A8


def trace(policy, num_steps, tower="generation"):
    return [step_mode(policy, tower, i, num_steps) for i in range(num_steps)]
